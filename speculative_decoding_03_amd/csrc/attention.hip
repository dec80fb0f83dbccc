// Grouped-query attention over the contiguous KV cache, for the K+1 verify rows (causal among
// the new rows, full over the committed prefix) and for the drafter's cross-attention into the
// target's cache (keys [0, len), no cache of its own).
//
// Split over keys (flash-decoding): grid (chunk, kv head, sequence); a workgroup of four waves
// takes one chunk of CH keys, each wave a contiguous quarter, and serves every query vector
// that reads that KV head (all rows x the group's query heads).  K is stored [pos][hd] and V
// transposed [hd][pos], so both MFMA operands stream as 16-byte loads.  Per chunk the kernel
// leaves (row max, sum of exponentials, unnormalised value sum); attn_combine merges the chunks
// in chunk order.  Chunk boundaries sit at fixed absolute positions and every reduction has a
// fixed order, so a row's output does not depend on how many other rows are in the call.

#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace specdec {

namespace {

constexpr int NWAVE = 4;

// Keys per wave: one 32-key block (measured on MI355X at the 31B shape: more workgroups and
// two waves per SIMD beat two blocks per wave at one wave per SIMD).
template <int HD> struct AttnShape {
  static constexpr int KPW = 32;  // keys per wave (one block: registers for 2 waves per SIMD)
  static constexpr int CH = KPW * NWAVE;            // keys per workgroup = one partial
  static constexpr int NB = KPW / 32;               // 32-key blocks per wave
  static constexpr int DS = (HD + 31) / 32;         // 32-wide head-dim steps (scores)
  static constexpr int DT = HD / 16;                // 16-row head-dim tiles (value sum)
  static constexpr int PST = HD + 4;                // partial row: o[HD], m, l, 2 pad
};

// Zeroes the elements of a fragment from index n on (its 8 elements are consecutive keys).
template <typename T>
__device__ __forceinline__ void keep_first(Frag<T>& f, int n) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.v[i] &= (2 * i < n ? 0x0000ffffu : 0u) | (2 * i + 1 < n ? 0xffff0000u : 0u);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) f.v[h][i] = 4 * h + i < n ? f.v[h][i] : 0u;
  }
}

// One workgroup = CH consecutive keys of one KV head of one sequence; wave w owns keys
// [chunk*CH + w*KPW, +KPW), which it loads once into registers.  Then, for each 16-vector tile of
// the group's query vectors (rows x query heads of the KV head), per wave:
//   S^T = K Q^T on MFMA (A = key rows, B = query vectors, k = head dim).  Key tile pairs map C
//   row i to key 8*(i/4) + i%4 (+4 in the second tile of the pair), so a lane's eight scores of
//   a query column are eight consecutive keys;
//   masked softmax statistics over the wave's keys per query column (max, then the sum of
//   exponentials; lanes combined by a fixed butterfly);
//   O^T = V^T P^T on MFMA with P^T taken straight from the score registers (bf16) and V^T read
//   from the transposed cache as 16-byte runs of the same eight keys.
// The four waves then merge through LDS (common max, rescale, sum in wave order) and wave 0
// writes the chunk's partial (o, m, l).  Keys that no row may see are never loaded.
template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
  using SH = AttnShape<HD>;
  constexpr int NB = SH::NB, DS = SH::DS, DT = SH::DT, KPW = SH::KPW, CH = SH::CH;
  __shared__ __align__(16) float xch[NWAVE - 1][16][SH::PST];
  __shared__ float mw[NWAVE][16], lw[NWAVE][16];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;

  const int len = a.len[b];
  const int end_max = len + a.R - 1 + a.key_off;  // keys [0, end_max) are read by some row
  if (end_max > a.max_ctx || len < 0) {
    if (chunk == 0 && g == 0 && threadIdx.x == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  if (chunk * CH >= end_max) return;  // uniform over the workgroup
  const int kw0 = chunk * CH + w * KPW;
  const T* Kc = reinterpret_cast<const T*>(a.kcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * a.max_ctx * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vcache) + (size_t)b * a.cache_b_stride +
                (size_t)g * HD * a.max_ctx;

  // ---- loads, without per-lane branches: K rows and the first query tile, then V^T runs ----
  // Addresses are clamped into the cache.  What a clamped or out-of-reach load brings in is
  // masked before use: scores of keys a row may not see become -inf, values past end_max zero.
  Frag<T> kf[NB][2][DS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = min(kw0 + nb * 32 + 8 * (c16 >> 2) + 4 * h + (c16 & 3), a.max_ctx - 1);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int d = ds * 32 + grp * 8;
        if (HD % 32 == 0 || d < HD) load_frag<T>(kf[nb][h][ds], Kc + (size_t)key * HD + d);
        else zero_frag(kf[nb][h][ds]);
      }
    }
  // this lane's query column of tile q0 (columns past Rall load a valid row; their scores are
  // masked to -inf), already in the storage type
  Frag<T> qf[DS];
  auto load_q = [&](int q0) {
    const int qc = min(q0 + c16, Rall - 1);
    const int row = qc / G;
    const T* qp = reinterpret_cast<const T*>(a.q) +
                  (((size_t)b * a.R + row) * a.hq + g * G + (qc - row * G)) * HD;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const int d = ds * 32 + grp * 8;
      if (HD % 32 == 0 || d < HD) load_frag<T>(qf[ds], qp + d);
      else zero_frag(qf[ds]);
    }
  };
  load_q(0);
  Frag<T> vf[NB][DT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int kk = min(kw0 + nb * 32 + grp * 8, a.max_ctx - 8);  // max_ctx is a multiple of 8
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) load_frag<T>(vf[nb][dt], Vt + (size_t)(dt * 16 + c16) * a.max_ctx + kk);
  }
  // every load above is issued before any instruction that waits for one of them
  __builtin_amdgcn_sched_barrier(0);
  const bool ragged = kw0 + KPW > end_max;  // the wave holds values past end_max (wave-uniform)

  float* pbase = a.part + (((size_t)b * a.hkv + g) * a.n_chunks + chunk) * (size_t)Rall * SH::PST;
  for (int q0 = 0; q0 < Rall; q0 += 16) {
    const int qv = q0 + c16;  // this lane's query column
    const int row = qv / G;

    // ---- scores, masked, and the softmax statistics of the wave's keys ----
    f32x4 s[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) acc = mma<T>(kf[nb][h][ds], qf[ds], acc);
        s[nb][h] = acc;
      }
    // the next tile's query vectors load while this tile finishes
    if (q0 + 16 < Rall) load_q(q0 + 16);
    const int kend = qv < Rall ? len + row + a.key_off : 0;  // keys [0, kend) are visible
    float m = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = kw0 + nb * 32 + 8 * grp + 4 * h + v;
          const float val = key < kend ? s[nb][h][v] * a.scale : -INFINITY;
          s[nb][h][v] = val;
          m = fmaxf(m, val);
        }
    m = fmaxf(m, __shfl_xor(m, 16, WAVE));
    m = fmaxf(m, __shfl_xor(m, 32, WAVE));
    float l = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float val = s[nb][h][v];
          const float p = val == -INFINITY ? 0.f : expf(val - m);
          s[nb][h][v] = p;
          l += p;
        }
    l += __shfl_xor(l, 16, WAVE);
    l += __shfl_xor(l, 32, WAVE);

    // ---- value sum O^T[d][q] = sum_key V^T[d][key] P^T[key][q] ----
    if (q0 == 0 && ragged) {  // values past end_max may hold anything, even NaN: zero them
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int nv = end_max - (kw0 + nb * 32 + grp * 8);  // visible elements of the lane's run
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) keep_first(vf[nb][dt], nv);
      }
    }
    Frag<T> pf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = s[nb][j >> 2][j & 3];
      to_frag<T>(pf[nb], y);
    }
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc = mma<T>(vf[nb][dt], pf[nb], acc);
      o[dt] = acc;
    }

    // ---- merge the four waves: common max, rescale, sum in wave order ----
    if (grp == 0) {
      mw[w][c16] = m;
      lw[w][c16] = l;
    }
    __syncthreads();
    float M = mw[0][c16];
#pragma unroll
    for (int u = 1; u < NWAVE; ++u) M = fmaxf(M, mw[u][c16]);
    const float f = m == -INFINITY ? 0.f : expf(m - M);
    if (w > 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(&xch[w - 1][c16][dt * 16 + 4 * grp]) = o[dt] * f;
    }
    __syncthreads();
    if (w == 0) {
      float L = 0.f;
#pragma unroll
      for (int u = 0; u < NWAVE; ++u) {
        const float mu = mw[u][c16];
        L += mu == -INFINITY ? 0.f : lw[u][c16] * expf(mu - M);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 y = o[dt] * f;
#pragma unroll
        for (int u = 0; u < NWAVE - 1; ++u)
          y += *reinterpret_cast<const f32x4*>(&xch[u][c16][dt * 16 + 4 * grp]);
        if (qv < Rall) *reinterpret_cast<f32x4*>(pbase + (size_t)qv * SH::PST + dt * 16 + 4 * grp) = y;
      }
      if (grp == 0 && qv < Rall) {
        pbase[(size_t)qv * SH::PST + HD] = M;
        pbase[(size_t)qv * SH::PST + HD + 1] = L;
      }
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
  // output element d of this query vector: row b*R + row, column h*hd + d of the O input
  T* const out = reinterpret_cast<T*>(a.out);
  const int orow = b * a.R + row, ocol = h * hd, ld = a.hq * hd;
  if (n_act == 0) {
    // no visible key (drafter before any context): the attention output is defined as zero
    for (int d = t; d < hd; d += blockDim.x)
      Elem<T>::store(out + x_offset(a.out_qx, orow, ocol + d, ld), 0.f);
    return;
  }
  const int pst = hd + 4;  // partial row: o[hd], m, l, 2 pad
  const size_t cstride = (size_t)Rall * pst;
  const float* pbase = a.part + ((size_t)b * a.hkv + g) * a.n_chunks * cstride + (size_t)qv * pst;
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
    Elem<T>::store(out + x_offset(a.out_qx, orow, ocol + t, ld), o * Linv);
  }
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  if (a.chunk != AttnShape<HD>::CH) return hipErrorInvalidValue;
  const int Rall = a.R * (a.hq / a.hkv);
  dim3 grid(a.n_launch, a.hkv, a.B), block(NWAVE * WAVE);
  hipLaunchKernelGGL((attn_kernel<T, HD>), grid, block, 0, st, a);
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

int attention_chunk(int head_dim) { return head_dim <= 128 ? AttnShape<128>::CH : AttnShape<256>::CH; }

bool attention_supported(int head_dim) {
  return head_dim == 64 || head_dim == 128 || head_dim == 176 || head_dim == 256;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.n_chunks > 4096 || a.n_launch < 1 || a.n_launch > a.n_chunks) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace specdec
