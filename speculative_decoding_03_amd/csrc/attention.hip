// Grouped-query attention over the contiguous KV cache, for the K+1 verify rows (causal among
// the new rows, full over the committed prefix) and for the drafter's cross-attention into the
// target's cache (keys [0, len), no cache of its own).
//
// Grid: (chunk, kv head, sequence).  A workgroup of 4 waves loads one chunk of CH keys of one
// KV head once and serves every query vector that reads that head (all rows x all query heads
// of the group, 16 per MFMA tile).  Scores S = Q K^T and the value sum P V both run on the
// 16x16x32 bf16 MFMA (fp32 storage: 16x16x4 fp32).  K is stored [pos][hd] and V transposed
// [hd][pos], so both operands stream as 16-byte loads along their reduction axis.  Per chunk the
// kernel leaves (row max, sum of exponentials, unnormalised value sum); attn_combine merges the
// chunks in chunk order.  Chunk boundaries sit at fixed absolute positions and every reduction
// has a fixed order, so a row's output does not depend on how many other rows are in the call.

#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace specdec {

namespace {

constexpr int NWAVE = 4;

template <int HD, int CH_> struct AttnShape {
  static constexpr int CH = CH_;                            // keys per chunk
  static constexpr int DS = (HD + 31) / 32;                 // 32-wide head-dim steps (scores)
  static constexpr int KB = CH / 16 / NWAVE;                // 16-key blocks per wave (scores)
  static constexpr int DB = (HD / 16 + NWAVE - 1) / NWAVE;  // 16-wide head-dim blocks per wave
  static constexpr int KS = CH / 32;                        // 32-key steps (values)
};

template <typename T, int HD, int QT, int CH_>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  using SH = AttnShape<HD, CH_>;
  constexpr int CH = SH::CH;
  __shared__ T pbuf[QT * 16 * CH];
  __shared__ float wred[NWAVE][QT * 16];
  __shared__ float mrow[QT * 16], lrow[QT * 16];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;
  const int key0 = chunk * CH;
  const T* Kc = reinterpret_cast<const T*>(a.kcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * a.max_ctx * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * HD * a.max_ctx;
  float* pbase = a.part + (((size_t)b * a.hkv + g) * a.n_chunks + chunk) * (size_t)Rall * (HD + 2);

  const int len = a.len[b];
  const int end_max = len + a.R - 1 + a.key_off;  // keys [0, end_max) are read by some row
  if (end_max > a.max_ctx || len < 0) {
    if (chunk == 0 && g == 0 && t == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  const int n_act = (end_max + CH - 1) / CH;
  if (chunk >= n_act) return;

  // The chunk's keys and values are loaded once, up front, and serve every query tile; values
  // of positions no row may see are zeroed (they may hold anything, even NaN).
  Frag<T> kf[SH::KB][SH::DS];
#pragma unroll
  for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
    for (int ds = 0; ds < SH::DS; ++ds) {
      const int key = key0 + (w + kb * NWAVE) * 16 + c16;
      const int d = ds * 32 + grp * 8;
      if (key < end_max && d < HD) load_frag<T>(kf[kb][ds], Kc + (size_t)key * HD + d);
      else zero_frag(kf[kb][ds]);
    }
  Frag<T> vf[SH::DB][SH::KS];
#pragma unroll
  for (int dbi = 0; dbi < SH::DB; ++dbi)
#pragma unroll
    for (int ks = 0; ks < SH::KS; ++ks) {
      const int db = w + dbi * NWAVE;
      const int kk = key0 + ks * 32 + grp * 8;
      const T* p = Vt + (size_t)(db * 16 + c16) * a.max_ctx + kk;
      if (db >= HD / 16 || kk >= end_max) {
        zero_frag(vf[dbi][ks]);
      } else if (kk + 8 <= end_max) {
        load_frag<T>(vf[dbi][ks], p);
      } else {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (kk + e < end_max) ? Elem<T>::load(p + e) : 0.f;
        to_frag<T>(vf[dbi][ks], y);
      }
    }
  auto load_q = [&](Frag<T> (&qf)[QT][SH::DS], int q0) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int qv = q0 + qt * 16 + c16;
      const int row = qv / G;
      const int h = g * G + (qv - row * G);
      const float* qp = a.q + (((size_t)b * a.R + row) * a.hq + h) * HD;
#pragma unroll
      for (int ds = 0; ds < SH::DS; ++ds) {
        const int d = ds * 32 + grp * 8;
        if (qv < Rall && d < HD) {
          const float4 x0 = *reinterpret_cast<const float4*>(qp + d);
          const float4 x1 = *reinterpret_cast<const float4*>(qp + d + 4);
          const float y[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          to_frag<T>(qf[qt][ds], y);
        } else {
          zero_frag(qf[qt][ds]);
        }
      }
    }
  };
  Frag<T> qf[QT][SH::DS];

  for (int q0 = 0; q0 < Rall; q0 += 16 * QT) {
    load_q(qf, q0);
    // ---- scores ----
    f32x4 s[QT][SH::KB];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < SH::DS; ++ds) acc = mma<T>(qf[qt][ds], kf[kb][ds], acc);
        s[qt][kb] = acc;
      }
    }
    // ---- softmax statistics of the chunk (fixed order: lanes, then waves) ----
    float M[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int qv = q0 + qt * 16 + grp * 4 + v;
        const int kend = len + qv / G + a.key_off;
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < SH::KB; ++kb) {
          const int key = key0 + (w + kb * NWAVE) * 16 + c16;
          const float val = (qv < Rall && key < kend) ? s[qt][kb][v] * a.scale : -INFINITY;
          s[qt][kb][v] = val;
          m = fmaxf(m, val);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
        if (c16 == 0) wred[w][qt * 16 + grp * 4 + v] = m;
      }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = qt * 16 + grp * 4 + v;
        M[qt][v] = fmaxf(fmaxf(wred[0][r], wred[1][r]), fmaxf(wred[2][r], wred[3][r]));
      }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < SH::KB; ++kb) {
          const float val = s[qt][kb][v];
          const float p = (val == -INFINITY) ? 0.f : expf(val - M[qt][v]);
          const int kl = (w + kb * NWAVE) * 16 + c16;
          Elem<T>::store(&pbuf[(qt * 16 + grp * 4 + v) * CH + kl], p);
          sum += p;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, WAVE);
        if (c16 == 0) wred[w][qt * 16 + grp * 4 + v] = sum;
      }
    __syncthreads();
    if (w == 0 && c16 == 0) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = qt * 16 + grp * 4 + v;
          mrow[r] = M[qt][v];
          lrow[r] = ((wred[0][r] + wred[1][r]) + wred[2][r]) + wred[3][r];
        }
    }
    // ---- values: O[qv][d] = sum_key P[qv][key] V[key][d] ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int dbi = 0; dbi < SH::DB; ++dbi) {
        const int db = w + dbi * NWAVE;
        if (db >= HD / 16) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < SH::KS; ++ks) {
          Frag<T> pf;
          load_frag<T>(pf, &pbuf[(qt * 16 + c16) * CH + ks * 32 + grp * 8]);
          acc = mma<T>(pf, vf[dbi][ks], acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int qv = q0 + qt * 16 + grp * 4 + v;
          if (qv < Rall) pbase[(size_t)qv * (HD + 2) + db * 16 + c16] = acc[v];
        }
      }
    }
    __syncthreads();
    if (t < QT * 16 && q0 + t < Rall) {
      pbase[(size_t)(q0 + t) * (HD + 2) + HD] = mrow[t];
      pbase[(size_t)(q0 + t) * (HD + 2) + HD + 1] = lrow[t];
    }
    __syncthreads();
  }
}

// Combines the chunk partials of one query vector:
// o = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c,  M = max_c m_c.
// Thread (p, d) sums chunks p, p+P, p+2P, ... of column d (P = 1024 / hd parts), and the P part
// sums are added in part order, so the result depends only on the chunk partials (a chunk whose
// keys are all invisible to the row contributes exact zeros).
template <typename T>
__global__ void __launch_bounds__(1024) attn_combine_kernel(AttnArgs a) {
  __shared__ float wts[4096];
  __shared__ float ls[4096];
  __shared__ float psum[1024];
  __shared__ float wmax[16];
  __shared__ float Linv;
  const int qv = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;
  const int hd = a.hd;
  const int len = a.len[b];
  const int end_max = len + a.R - 1 + a.key_off;
  if (end_max > a.max_ctx || len < 0) return;
  const int n_act = (end_max + a.chunk - 1) / a.chunk;
  if (n_act > a.n_launch) {  // the device length is beyond the host-side bound
    if (t == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  const int row = qv / G, h = g * G + (qv - row * G);
  T* out = reinterpret_cast<T*>(a.out) + ((size_t)b * a.R + row) * (a.hq * hd) + h * hd;
  if (n_act == 0) {
    // no visible key (drafter before any context): the attention output is defined as zero
    for (int d = t; d < hd; d += blockDim.x) Elem<T>::store(out + d, 0.f);
    return;
  }
  const size_t cstride = (size_t)Rall * (hd + 2);
  const float* pbase = a.part + ((size_t)b * a.hkv + g) * a.n_chunks * cstride + (size_t)qv * (hd + 2);
  // chunk max over (m_c): per-thread stripes, then waves in order
  float mx = -INFINITY;
  for (int c = t; c < n_act; c += blockDim.x) {
    const float2 ml = *reinterpret_cast<const float2*>(pbase + c * cstride + hd);
    wts[c] = ml.x;
    ls[c] = ml.y;
    mx = fmaxf(mx, ml.x);
  }
  mx = wave_max(mx);
  if ((t & 63) == 0) wmax[t >> 6] = mx;
  __syncthreads();
  float M = wmax[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) M = fmaxf(M, wmax[w]);
  for (int c = t; c < n_act; c += blockDim.x)
    wts[c] = (wts[c] == -INFINITY) ? 0.f : expf(wts[c] - M);
  __syncthreads();
  if (t == 0) {
    float L = 0.f;
    for (int c = 0; c < n_act; ++c) L += ls[c] * wts[c];
    Linv = 1.0f / L;
  }
  const int P = blockDim.x / hd;  // chunk parts
  const int p = t / hd, d = t - p * hd;
  float acc = 0.f;
  if (p < P) {
    int c = p;
    for (; c + 3 * P < n_act; c += 4 * P) {
      const float v0 = pbase[(size_t)c * cstride + d];
      const float v1 = pbase[(size_t)(c + P) * cstride + d];
      const float v2 = pbase[(size_t)(c + 2 * P) * cstride + d];
      const float v3 = pbase[(size_t)(c + 3 * P) * cstride + d];
      acc += wts[c] * v0;
      acc += wts[c + P] * v1;
      acc += wts[c + 2 * P] * v2;
      acc += wts[c + 3 * P] * v3;
    }
    for (; c < n_act; c += P) acc += wts[c] * pbase[(size_t)c * cstride + d];
    psum[p * hd + d] = acc;
  }
  __syncthreads();
  if (t < hd) {
    float o = psum[t];
    for (int q = 1; q < P; ++q) o += psum[q * hd + t];
    Elem<T>::store(out + t, o * Linv);
  }
}

template <typename T, int HD, int CH>
void launch_ch(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_launch, a.hkv, a.B), block(256);
  const int Rall = a.R * (a.hq / a.hkv);
  if (Rall <= 16)
    hipLaunchKernelGGL((attn_kernel<T, HD, 1, CH>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, HD, 2, CH>), grid, block, 0, st, a);
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  if constexpr (HD <= 128) {
    if (a.chunk == 256) launch_ch<T, HD, 256>(a, st);
    else if (a.chunk == 128) launch_ch<T, HD, 128>(a, st);
    else return hipErrorInvalidValue;
  } else {
    if (a.chunk != 128) return hipErrorInvalidValue;
    launch_ch<T, HD, 128>(a, st);
  }
  const int Rall = a.R * (a.hq / a.hkv);
  dim3 cgrid(Rall, a.hkv, a.B), cblock(1024);
  hipLaunchKernelGGL(attn_combine_kernel<T>, cgrid, cblock, 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  switch (a.hd) {
    case 64: return launch_hd<T, 64>(a, st);
    case 128: return launch_hd<T, 128>(a, st);
    case 176: return launch_hd<T, 176>(a, st);
    case 256: return launch_hd<T, 256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attention_chunk(int head_dim) {
  static const int forced = [] {
    const char* e = getenv("SPECDEC_ATTN_CHUNK");
    return e ? atoi(e) : 0;
  }();
  if (head_dim <= 128 && (forced == 128 || forced == 256)) return forced;
  return 128;
}

bool attention_supported(int head_dim) {
  return head_dim == 64 || head_dim == 128 || head_dim == 176 || head_dim == 256;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.n_chunks > 4096 || a.n_launch < 1 || a.n_launch > a.n_chunks) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace specdec
