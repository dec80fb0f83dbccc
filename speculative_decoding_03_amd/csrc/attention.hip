// Grouped-query attention over the contiguous KV cache, for the K+1 verify rows (causal among
// the new rows, full over the committed prefix) and for the drafter's cross-attention into the
// target's cache (keys [0, len), no cache of its own).
//
// Split over keys (flash-decoding): grid (chunk, kv head, sequence x query tiles); a workgroup of
// NW waves (four, or two for models with few KV heads) takes one chunk of CH = 32 NW keys, each
// wave a contiguous 32-key block, and serves every query vector that reads that KV head (all rows
// x the group's query heads), or one 16-vector tile of them when the call splits its tiles over
// workgroups.  K is stored [pos][hd] and V transposed [hd][pos], so both MFMA operands stream as
// 16-byte loads.  Per chunk the kernel leaves (row max in base-2 units, sum of exponentials,
// unnormalised value sum); attn_combine merges the chunks in chunk order.  The value sums are kept in the storage type (bf16 rounds
// each chunk's sum once, well inside the bf16 path's error budget, and halves the partial
// traffic); the maxima and sums of exponentials stay fp32.  Chunk boundaries sit at fixed
// absolute positions and every reduction has a fixed order, so a row's output does not depend
// on how many other rows are in the call.

#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace specdec {

namespace {

// Keys per wave: one 32-key block (measured on MI355X at the 31B shape: more workgroups and
// two waves per SIMD beat two blocks per wave at one wave per SIMD).
template <int HD, int NW> struct AttnShape {
  static constexpr int KPW = 32;  // keys per wave (one block: registers for 2 waves per SIMD)
  static constexpr int CH = KPW * NW;               // keys per workgroup = one partial
  static constexpr int NB = KPW / 32;               // 32-key blocks per wave
  static constexpr int DS = (HD + 31) / 32;         // 32-wide head-dim steps (scores)
  static constexpr int DT = HD / 16;                // 16-row head-dim tiles (value sum)
  static constexpr int PST = HD + 4;                // partial row: o[HD], m, l, 2 pad
};

// Waves per SIMD the register allocation must allow.  Three for 16-bit heads of up to 128: a
// 31B-class layer at 8K context launches 65 chunks x 8 KV heads = 2080 waves, just over the
// 2048 slots that two waves per SIMD give on 256 CUs, and the few left over would otherwise run
// as a second round after the first has drained.  Larger heads keep the compiler's choice.
template <typename T, int HD> constexpr int attn_occupancy() {
  return sizeof(T) == 2 && HD <= 128 ? 3 : 1;
}

// 2^x on the hardware exponential (2^-inf = 0).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48), on the gfx950
// row-swap instructions: after a swap the pair (first, second) holds both rows' values in every
// lane, in the same order, so every lane of a group ends with the same bits.
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// A chunk partial row: the value sum o[HD] in the storage type at the start of the row, then
// (m, l) in fp32 at float offset HD; rows are HD + 4 floats apart.
template <typename T>
__device__ __forceinline__ void store_part_o(float* row, int d0, const f32x4& y) {
  if constexpr (sizeof(T) == 2) {
    const uint2 pk = {f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(row) + d0) = pk;
  } else {
    *reinterpret_cast<f32x4*>(row + d0) = y;
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
// The NW waves then merge through LDS (common max, rescale, sum in wave order), each wave
// writing 1/NW of the chunk's partial (o, m, l).  Exponentials are 2^x on the hardware
// instruction, with scores scaled by scale * log2 e.  Keys that no row may see are never loaded.
template <typename T, int HD, int NW, bool TREE>
__global__ void __launch_bounds__(NW * WAVE) __attribute__((amdgpu_waves_per_eu(attn_occupancy<T, HD>())))
attn_kernel(AttnArgs a) {
  using SH = AttnShape<HD, NW>;
  constexpr int NB = SH::NB, DS = SH::DS, DT = SH::DT, KPW = SH::KPW, CH = SH::CH;
  __shared__ __align__(16) float xch[NW][16][SH::PST];
  __shared__ float mw[NW][16], lw[NW][16];
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;
  // query vectors [q_begin, q_end) of the group: all of them, or tile blockIdx.z % nqt
  const int nqt = a.q_split ? (Rall + 15) / 16 : 1;
  const int b = blockIdx.z / nqt;
  const int q_begin = (blockIdx.z - b * nqt) * 16;
  const int q_end = a.q_split ? min(Rall, q_begin + 16) : Rall;
  const float scale2 = a.scale * 1.44269504088896341f;  // softmax scale times log2 e

  // The committed length is requested first but waited for only after every cache and query
  // load is in flight: no load address depends on it (each is clamped into the cache), so its
  // latency overlaps theirs.  A chunk launched past the visible keys returns after its loads.
  const int len_in = a.len[b];
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
  Frag<T> qa[DS], qb[DS];
  auto load_q = [&](int q0, Frag<T> (&qf)[DS]) {
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
  load_q(q_begin, qa);
  if (q_begin + 16 < q_end) load_q(q_begin + 16, qb);  // the second tile's, requested up front
  Frag<T> vf[NB][DT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int kk = min(kw0 + nb * 32 + grp * 8, a.max_ctx - 8);  // max_ctx is a multiple of 8
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) load_frag<T>(vf[nb][dt], Vt + (size_t)(dt * 16 + c16) * a.max_ctx + kk);
  }
  // every load above is issued before any instruction that waits for one of them
  __builtin_amdgcn_sched_barrier(0);
  const int len = len_in;
  const int end_max = attn_key_end(a.vis, len, a.R, a.key_off);  // keys some row may see
  if (end_max > a.max_ctx || len < 0) {
    if (chunk == 0 && g == 0 && threadIdx.x == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  if (chunk * CH >= end_max) return;  // uniform over the workgroup
  const bool ragged = kw0 + KPW > end_max;  // the wave holds values past end_max (wave-uniform)

  float* pbase = a.part + (((size_t)b * a.hkv + g) * a.n_chunks + chunk) * (size_t)Rall * SH::PST;
  bool v_clean = !ragged;  // values past end_max zeroed (done once, by the first tile that uses them)
  auto tile = [&](int q0, Frag<T> (&qf)[DS]) {
    const int qv = q0 + c16;  // this lane's query column
    const int row = qv / G;
    // causal rows that all end before this chunk: no partial is needed (the combine reads a
    // row's chunks only up to its own last key); uniform over the workgroup
    if (a.vis == VIS_CAUSAL && chunk * CH >= len + min(q0 + 15, Rall - 1) / G + a.key_off) {
      if (q0 + 32 < q_end) load_q(q0 + 32, qf);
      return;
    }

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
    // the tile after next reuses this tile's buffer once its scores are done
    if (q0 + 32 < q_end) load_q(q0 + 32, qf);
    // keys [0, kend) are visible, and in a tree verify slot len + j for each bit j of tmask
    const int kend = qv >= Rall ? 0 : (a.vis == VIS_CAUSAL ? len + row + a.key_off
                                                           : (a.vis == VIS_FLAT ? len + a.key_off : len));
    uint64_t tmask = 0ull;
    if constexpr (TREE) tmask = qv < Rall ? a.tree_mask[row] : 0ull;
    // scores in base-2 units (scale * log2 e folded in): exp(x - m) = exp2(x2 - m2)
    float m = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = kw0 + nb * 32 + 8 * grp + 4 * h + v;
          bool vis = key < kend;
          if constexpr (TREE) {
            const unsigned tj = (unsigned)(key - len);  // slot of a tree node (when < 64)
            vis |= tj < 64u && ((tmask >> tj) & 1ull);
          }
          const float val = vis ? s[nb][h][v] * scale2 : -INFINITY;
          s[nb][h][v] = val;
          m = fmaxf(m, val);
        }
    m = rows_max(m);
    // a column with no visible key keeps m = -inf; its exponentials are exp2(-inf) = 0
    const float ms = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = exp2_hw(s[nb][h][v] - ms);
          s[nb][h][v] = p;
          l += p;
        }
    l = rows_sum(l);

    // ---- value sum O^T[d][q] = sum_key V^T[d][key] P^T[key][q] ----
    if (!v_clean) {  // values past end_max may hold anything, even NaN: zero them
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int nv = end_max - (kw0 + nb * 32 + grp * 8);  // visible elements of the lane's run
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) keep_first(vf[nb][dt], nv);
      }
      v_clean = true;
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

    // ---- merge the NW waves: common max, rescale, sum in wave order ----
    // Every wave parks its statistics and unscaled sums in LDS; after one barrier wave w
    // rescales and adds up head-dim tiles w, w+NW, ... over the NW waves (in wave order) and
    // writes them to the partial.
    if (grp == 0) {
      mw[w][c16] = m;
      lw[w][c16] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(&xch[w][c16][dt * 16 + 4 * grp]) = o[dt];
    __syncthreads();
    float mu[NW], fu[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u) mu[u] = mw[u][c16];
    float M = mu[0];
#pragma unroll
    for (int u = 1; u < NW; ++u) M = fmaxf(M, mu[u]);
    const float Ms = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int u = 0; u < NW; ++u) fu[u] = exp2_hw(mu[u] - Ms);  // 0 for a wave with no key
#pragma unroll
    for (int dt = w; dt < DT; dt += NW) {
      f32x4 y = *reinterpret_cast<const f32x4*>(&xch[0][c16][dt * 16 + 4 * grp]) * fu[0];
#pragma unroll
      for (int u = 1; u < NW; ++u)
        y += *reinterpret_cast<const f32x4*>(&xch[u][c16][dt * 16 + 4 * grp]) * fu[u];
      if (qv < Rall) store_part_o<T>(pbase + (size_t)qv * SH::PST, dt * 16 + 4 * grp, y);
    }
    if (w == 0 && grp == 0 && qv < Rall) {
      float L = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) L += lw[u][c16] * fu[u];
      pbase[(size_t)qv * SH::PST + HD] = M;
      pbase[(size_t)qv * SH::PST + HD + 1] = L;
    }
    if (q0 + 16 < q_end) __syncthreads();  // the next tile reuses the LDS buffers
  };
  for (int q0 = q_begin; q0 < q_end; q0 += 32) {
    tile(q0, qa);
    if (q0 + 16 < q_end) tile(q0 + 16, qb);
  }
}

// Combines the chunk partials of one query vector on one wave:
// o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c (maxima in base-2 units).
// A partial row's value sum is read as 16-byte runs: lane (r, q) = (lane % RN, lane / RN) takes
// run r of chunks q, q + QN, q + 2 QN, ... (QN = 64 / RN chunk groups).  Each lane requests a
// batch of CB chunks (value run and (m, l)) before it uses any of them, keeps a running maximum
// of its own chunks and rescales its sums when the maximum grows, then the QN groups are merged
// through LDS in group order.  Chunk c always belongs to the same lane and batch, so the result
// depends only on the row's own partials (a chunk whose keys the row cannot see has m = -inf and
// adds exact zeros).
template <typename T, int HD>
__global__ void __launch_bounds__(WAVE) attn_combine_kernel(AttnArgs a) {
  constexpr int EPR = 16 / (int)sizeof(T);  // elements per 16-byte run
  constexpr int RN = HD / EPR;              // runs per partial row
  constexpr int QN = WAVE / RN;             // chunk groups
  // chunks per lane per batch: at head size 128, 96 chunks (12K keys in 128-key chunks) in one batch
  constexpr int CB = 24;
  static_assert(HD % EPR == 0 && RN <= WAVE && QN >= 1, "partial row does not fit a wave");
  __shared__ __align__(16) float red[QN][HD];
  __shared__ float lred[QN];
  const int qv = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int row = qv / G, h = g * G + (qv - row * G);
  T* const out = reinterpret_cast<T*>(a.out);
  const int orow = b * a.R + row, ocol = h * HD, ld = a.hq * HD;
  const int r = lane % RN, q = lane / RN;
  const bool active = q < QN;
  const int pst = HD + 4;  // partial row: o[HD] (storage type), then (m, l) fp32 at float HD
  const size_t cstride = (size_t)a.R * G * pst;
  const float* pbase = a.part + ((size_t)b * a.hkv + g) * a.n_chunks * cstride + (size_t)qv * pst;
  // Batches cover the chunks the launch may have written (the host-side bound n_launch), so the
  // first batch's loads are in flight before the committed length arrives; chunks past the
  // row's visible ones (n_act) are loaded but never used.
  const int len_in = a.len[b];
  float mq = -INFINITY, lq = 0.f, acc[EPR];
#pragma unroll
  for (int e = 0; e < EPR; ++e) acc[e] = 0.f;
  const int per_lane = (a.n_launch + QN - 1) / QN;  // chunks of the busiest group
  int n_act = -1;
  for (int k0 = 0; k0 < per_lane; k0 += CB) {
    u32x4 ov[CB];
    float2 ml[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      // a chunk past the launch reads chunk 0 again (in bounds) and is not used
      const int c = q + QN * (k0 + k);
      const float* rowp = pbase + (size_t)(active && c < a.n_launch ? c : 0) * cstride;
      ov[k] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(rowp) + r * 16);
      ml[k] = *reinterpret_cast<const float2*>(rowp + HD);
    }
    if (n_act < 0) {
      const int len = len_in;
      const int end_max = attn_key_end(a.vis, len, a.R, a.key_off);
      if (end_max > a.max_ctx || len < 0) return;
      if ((end_max + a.chunk - 1) / a.chunk > a.n_launch) {  // beyond the host-side bound
        if (lane == 0) raise_error(a.err, ERRBIT_CAPACITY);
        return;
      }
      // the chunks that hold a key this row sees (a causal row ends at its own key; chunks
      // after it, which only later rows see, contribute exact zeros and are not read)
      const int row_end = a.vis == VIS_CAUSAL ? len + row + a.key_off : end_max;
      n_act = (row_end + a.chunk - 1) / a.chunk;
      if (n_act == 0) {
        // no visible key (drafter before any context): the attention output is defined as zero
        if (active && q == 0)
          *reinterpret_cast<u32x4*>(out + x_offset(a.out_qx, orow, ocol + r * EPR, ld)) = u32x4{0, 0, 0, 0};
        return;
      }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < CB; ++k)
      if (active && q + QN * (k0 + k) < n_act) mb = fmaxf(mb, ml[k].x);
    const float mn = fmaxf(mq, mb);
    if (mn != mq) {  // the running maximum grew: rescale what this lane has summed
      const float sc = exp2_hw(mq - mn);  // mq = -inf: sums are zero, 2^-inf = 0
#pragma unroll
      for (int e = 0; e < EPR; ++e) acc[e] *= sc;
      lq *= sc;
      mq = mn;
    }
    const float ms = mq == -INFINITY ? 0.f : mq;
#pragma unroll
    for (int k = 0; k < CB; ++k) {
      if (!(active && q + QN * (k0 + k) < n_act)) continue;
      const float w = exp2_hw(ml[k].x - ms);
      lq += w * ml[k].y;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w * __uint_as_float(ov[k][i] << 16);
          acc[2 * i + 1] += w * __uint_as_float(ov[k][i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += w * __uint_as_float(ov[k][i]);
      }
    }
  }
  // merge the chunk groups in group order, each rescaled to the common maximum
  const float M = wave_max(active ? mq : -INFINITY);
  const float Ms = M == -INFINITY ? 0.f : M;
  const float f = exp2_hw(mq - Ms);  // a group that saw no key: 2^-inf = 0
  if (active) {
#pragma unroll
    for (int e = 0; e < EPR; ++e) red[q][r * EPR + e] = acc[e] * f;
    if (r == 0) lred[q] = lq * f;
  }
  __syncthreads();
  if (active && q == 0) {
    float L = lred[0];
#pragma unroll
    for (int u = 1; u < QN; ++u) L += lred[u];
    const float inv = 1.0f / L;
    float o[EPR];
#pragma unroll
    for (int e = 0; e < EPR; ++e) {
      o[e] = red[0][r * EPR + e];
#pragma unroll
      for (int u = 1; u < QN; ++u) o[e] += red[u][r * EPR + e];
      o[e] *= inv;
    }
    // the run's EPR elements are consecutive in the output (row-major or quad layout)
    u32x4 pk;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = f32x2_to_bf16x2(o[2 * i], o[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = __float_as_uint(o[i]);
    }
    *reinterpret_cast<u32x4*>(out + x_offset(a.out_qx, orow, ocol + r * EPR, ld)) = pk;
  }
}

// Prompt attention: the rows of a prompt chunk of one sequence (causal, over the committed prefix
// and the chunk), bf16.  A workgroup of NWQ waves takes 16 * NWQ consecutive query vectors of one
// KV head (rows x the group's query heads) and walks every key any of them sees in steps of KS
// keys.  Each step's K rows and V^T runs are copied from the cache into LDS in MFMA operand order
// (a fragment = 64 lanes x 16 bytes, one run per thread and fragment, conflict-free), with the
// values of keys past the block's last visible key zeroed as they are stored; every wave then
// multiplies its 16 query vectors against the step on MFMA (S^T = K Q^T, O^T += V^T P^T with P^T
// taken from the score registers, as in attn_kernel) under an online softmax: the running
// maximum in base-2 units, and the sums rescaled by 2^(m_old - m_new) when it grows.  The output
// is normalised and stored directly.  With n_chunks > 1 the keys are split into n_chunks ranges
// of `chunk` keys (grid z): each workgroup leaves a chunk partial of its range in attn_kernel's
// format and attn_combine_kernel merges the ranges.  Two LDS stages alternate; the next step's
// loads are in flight while the current one is multiplied.
template <int HD, int NWQ, int QT>
__global__ void __launch_bounds__(NWQ * 64) attn_prompt_kernel(AttnArgs a) {
  using T = bf16_t;
  constexpr int KS = HD <= 128 ? 64 : 32;  // keys per step
  constexpr int NB = KS / 32;              // 32-key blocks per step
  constexpr int DS = HD / 32, DT = HD / 16;
  constexpr int KFR = NB * 2 * DS, VFR = NB * DT;  // K and V^T fragments per step
  constexpr int NTH = NWQ * 64;
  constexpr int KR = KFR * 64 / NTH, VR = VFR * 64 / NTH;  // runs per thread and step
  static_assert(HD % 32 == 0 && KFR * 64 % NTH == 0 && VFR * 64 % NTH == 0, "step layout");
  __shared__ __align__(16) u32x4 sk[2][KFR * 64];
  __shared__ __align__(16) u32x4 sv[2][VFR * 64];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, grp = lane >> 4;
  const int g = blockIdx.y;
  const int G = a.hq / a.hkv;
  const int Rall = a.R * G;
  const int v_blk = blockIdx.x * 16 * NWQ * QT;
  const float scale2 = a.scale * 1.44269504088896341f;
  const int len = a.len[0];
  // keys [0, kend_blk) hold every key a row of the block sees
  const int row_last = (min(v_blk + 16 * NWQ * QT, Rall) - 1) / G;
  const int kend_blk = len + row_last + a.key_off;
  if (kend_blk > a.max_ctx || len < 0) {
    if (blockIdx.x == 0 && g == 0 && tid == 0) raise_error(a.err, ERRBIT_CAPACITY);
    return;
  }
  // this workgroup's key range
  const int kr0 = blockIdx.z * a.chunk;
  const int kr1 = a.n_chunks > 1 ? min(kend_blk, kr0 + a.chunk) : kend_blk;
  if (kr0 >= kend_blk) return;  // no row of the block sees the range (the combine reads none)
  const int n_steps = (kr1 - kr0 + KS - 1) / KS;
  const T* Kc = reinterpret_cast<const T*>(a.kcache) + (size_t)g * a.max_ctx * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vcache) + (size_t)g * HD * a.max_ctx;

  // this wave's QT tiles of 16 query vectors (a vector past Rall loads a valid one; it is
  // never stored)
  int qv[QT], qrow[QT], kend[QT];  // kend: keys the lane's query vector of tile t sees
  Frag<T> qf[QT][DS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    qv[t] = v_blk + 16 * (w * QT + t) + c16;
    const int qc = min(qv[t], Rall - 1);
    qrow[t] = qc / G;
    kend[t] = len + qrow[t] + a.key_off;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)qrow[t] * a.hq + g * G + (qc - qrow[t] * G)) * HD;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) load_frag<T>(qf[t][ds], qp + ds * 32 + grp * 8);
  }

  // the thread's runs of a step: run i = tid + j * NTH is lane i % 64 of fragment i / 64
  u32x4 rk[KR], rv[VR];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int i = tid + j * NTH, f = i / 64, ln = i % 64;
      const int nb = f / (2 * DS), h = (f / DS) % 2, ds = f % DS;
      const int lc = ln & 15, lg = ln >> 4;
      const int key = min(k0 + nb * 32 + 8 * (lc >> 2) + 4 * h + (lc & 3), a.max_ctx - 1);
      rk[j] = *reinterpret_cast<const u32x4*>(Kc + (size_t)key * HD + ds * 32 + lg * 8);
    }
#pragma unroll
    for (int j = 0; j < VR; ++j) {
      const int i = tid + j * NTH, f = i / 64, ln = i % 64;
      const int nb = f / DT, dt = f % DT;
      const int lc = ln & 15, lg = ln >> 4;
      const int kk = min(k0 + nb * 32 + lg * 8, a.max_ctx - 8);  // max_ctx is a multiple of 8
      rv[j] = *reinterpret_cast<const u32x4*>(Vt + (size_t)(dt * 16 + lc) * a.max_ctx + kk);
    }
  };
  auto store_step = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < KR; ++j) sk[buf][tid + j * NTH] = rk[j];
#pragma unroll
    for (int j = 0; j < VR; ++j) {
      const int i = tid + j * NTH, f = i / 64, ln = i % 64;
      const int nb = f / DT;
      Frag<T> fr;
      fr.v = rv[j];
      keep_first(fr, kend_blk - (k0 + nb * 32 + (ln >> 4) * 8));  // values past the block's keys
      sv[buf][i] = fr.v;
    }
  };

  // the fewest keys any query vector of the wave sees: a step below it needs no causal mask
  int kend_min = kend[0];
#pragma unroll
  for (int t = 1; t < QT; ++t) kend_min = min(kend_min, kend[t]);
  kend_min = (int)-wave_max(-(float)kend_min);  // key counts are exact in fp32
  float m_run[QT], l_lane[QT];
  f32x4 o[QT][DT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_lane[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](int buf, int k0) {
    const bool full = k0 + KS <= kend_min;  // every key of the step is visible (wave-uniform)
    float sc[QT][NB][8];
    float mb[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) mb[t] = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          Frag<T> kf;
          kf.v = sk[buf][((nb * 2 + h) * DS + ds) * 64 + lane];
#pragma unroll
          for (int t = 0; t < QT; ++t) acc[t] = mma<T>(kf, qf[t][ds], acc[t]);
        }
#pragma unroll
        for (int t = 0; t < QT; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int key = k0 + nb * 32 + 8 * grp + 4 * h + v;
            const float val = (full || key < kend[t]) ? acc[t][v] * scale2 : -INFINITY;
            sc[t][nb][4 * h + v] = val;
            mb[t] = fmaxf(mb[t], val);
          }
      }
    float ms[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const float mn = fmaxf(m_run[t], rows_max(mb[t]));
      ms[t] = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2_hw(m_run[t] - ms[t]);  // m_run = -inf: 0 (nothing summed yet)
      // a factor of exactly 1 (no column's maximum grew) leaves the sums as they are
      if (__ballot(alpha != 1.0f) != 0ull) {
        l_lane[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
      }
      m_run[t] = mn;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      Frag<T> pf[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          y[j] = exp2_hw(sc[t][nb][j] - ms[t]);
          l_lane[t] += y[j];
        }
        to_frag<T>(pf[t], y);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        Frag<T> vf;
        vf.v = sv[buf][(nb * DT + dt) * 64 + lane];
#pragma unroll
        for (int t = 0; t < QT; ++t) o[t][dt] = mma<T>(vf, pf[t], o[t][dt]);
      }
    }
  };

  load_step(kr0);
  for (int s = 0; s < n_steps; ++s) {
    const int k0 = kr0 + s * KS;
    store_step(s & 1, k0);
    if (s + 1 < n_steps) load_step(k0 + KS);
    __syncthreads();
    compute(s & 1, k0);
  }

  // normalise and store: lane (grp, c16) holds head-dim elements dt*16 + 4*grp .. +3 of its vector
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float lsum = rows_sum(l_lane[t]);
    if (qv[t] >= Rall) continue;
    if (a.n_chunks > 1) {  // the range's partial: unnormalised sums, then (max, sum) in fp32
      float* row = a.part + ((size_t)g * a.n_chunks + blockIdx.z) * (size_t)Rall * (HD + 4) +
                   (size_t)qv[t] * (HD + 4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store_part_o<T>(row, dt * 16 + 4 * grp, o[t][dt]);
      if (grp == 0) {
        row[HD] = m_run[t];
        row[HD + 1] = lsum;
      }
    } else {
      const float inv = 1.0f / lsum;
      T* out = reinterpret_cast<T*>(a.out) + (size_t)qrow[t] * a.hq * HD +
               (size_t)(g * G + (qv[t] - qrow[t] * G)) * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 pk = {f32x2_to_bf16x2(o[t][dt][0] * inv, o[t][dt][1] * inv),
                          f32x2_to_bf16x2(o[t][dt][2] * inv, o[t][dt][3] * inv)};
        *reinterpret_cast<uint2*>(out + dt * 16 + 4 * grp) = pk;
      }
    }
  }
}

template <typename T, int HD, int NW>
void launch_nw(const AttnArgs& a, dim3 grid, hipStream_t st) {
  if (a.vis == VIS_TREE)
    hipLaunchKernelGGL((attn_kernel<T, HD, NW, true>), grid, dim3(NW * WAVE), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, HD, NW, false>), grid, dim3(NW * WAVE), 0, st, a);
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  if (a.vis == VIS_TREE && !a.tree_mask) return hipErrorInvalidValue;
  const int Rall = a.R * (a.hq / a.hkv);
  const int nqt = a.q_split ? (Rall + 15) / 16 : 1;
  dim3 grid(a.n_launch, a.hkv, a.B * nqt);
  if (a.chunk == AttnShape<HD, 4>::CH) launch_nw<T, HD, 4>(a, grid, st);
  else if (a.chunk == AttnShape<HD, 2>::CH) launch_nw<T, HD, 2>(a, grid, st);
  else return hipErrorInvalidValue;
  dim3 cgrid(Rall, a.hkv, a.B), cblock(WAVE);
  hipLaunchKernelGGL((attn_combine_kernel<T, HD>), cgrid, cblock, 0, st, a);
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

int attention_chunk(int n_kv_heads, int max_ctx) {
  // 64-key chunks (two-wave workgroups) when 128-key ones give fewer than 64 workgroups even at the
  // longest context.  Measured on MI355X (attention + combine, one sequence): a single KV head of
  // 256 at 2K context, 4 rows 14.4 -> 11.9 us and 1 row 11.3 -> 9.6 us; two KV heads at 4K no
  // change; four KV heads of 176 at 4K and eight of 128 at 8K 1.5-2.3 us slower.
  return n_kv_heads * ((max_ctx + 127) / 128) < 64 ? AttnShape<128, 2>::CH : AttnShape<128, 4>::CH;
}

bool attention_q_split(int n_launch, int hkv, int B, int R, int G) {
  // one query tile per workgroup when a launch has more than one tile and fewer than 128
  // workgroups.  Measured on MI355X: 4-5 rows x 8 query heads of a single KV head at 2K context
  // (33 workgroups) 11.9 -> 10.0 us, two KV heads at 4K (66) 14.3 -> 12.2 us; with 132 or more
  // workgroups (four KV heads at 4K, eight at 8K) it is 0.6-2 us slower.
  return R * G > 16 && n_launch * hkv * B < 128;
}

bool attention_supported(int head_dim) {
  return head_dim == 64 || head_dim == 128 || head_dim == 176 || head_dim == 256;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.n_chunks > 4096 || a.n_launch < 1 || a.n_launch > a.n_chunks) return hipErrorInvalidValue;
  return dtype == DT_BF16 ? launch_t<bf16_t>(a, st) : launch_t<float>(a, st);
}

// query tiles per wave (measured on MI355X, 31B and E2B prompts of 512 rows: two tiles, which
// share each LDS fragment read but need 223 registers, are 4-6% slower than one)
constexpr int PROMPT_QT = 1;
// Combines the key-range partials of a prompt's query vectors (at most PROMPT_COMBINE_RANGES
// ranges, B = 1): HD / 8 lanes per vector, each a 16-byte run of the head dimension, read the
// vector's ranges that hold a key its row sees (later ranges may hold no partial) and form
// o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c, M = max_c m_c, with no exchange between lanes.
constexpr int PROMPT_COMBINE_RANGES = 4;
template <int HD>
__global__ void __launch_bounds__(256) attn_combine_few_kernel(AttnArgs a) {
  constexpr int SUB = HD / 8;     // lanes per query vector
  constexpr int VPB = 256 / SUB;  // query vectors per workgroup
  constexpr int NR = PROMPT_COMBINE_RANGES;
  const int G = a.hq / a.hkv, Rall = a.R * G;
  const int qv = blockIdx.x * VPB + (int)threadIdx.x / SUB, r = threadIdx.x % SUB, g = blockIdx.y;
  if (qv >= Rall) return;
  const int len = a.len[0];
  const int row = qv / G, h = g * G + (qv - row * G);
  const int row_end = len + row + a.key_off;  // the row sees keys [0, row_end)
  if (len < 0 || row_end > a.max_ctx) return;  // flagged by the attention launch
  const int n_act = min(a.n_chunks, (row_end + a.chunk - 1) / a.chunk);
  const size_t pst = HD + 4, cstride = (size_t)Rall * pst;
  const float* pbase = a.part + (size_t)g * a.n_chunks * cstride + (size_t)qv * pst;
  u32x4 ov[NR];
  float m[NR], l[NR];
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    if (c < n_act) {
      const float* rowp = pbase + (size_t)c * cstride;
      ov[c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(rowp) + r * 16);
      const float2 ml = *reinterpret_cast<const float2*>(rowp + HD);
      m[c] = ml.x;
      l[c] = ml.y;
    } else {
      ov[c] = u32x4{0, 0, 0, 0};
      m[c] = -INFINITY;
      l[c] = 0.f;
    }
  }
  float M = m[0];
#pragma unroll
  for (int c = 1; c < NR; ++c) M = fmaxf(M, m[c]);
  const float Ms = M == -INFINITY ? 0.f : M;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, L = 0.f;
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const float w = exp2_hw(m[c] - Ms);  // a range the row does not see: 2^-inf = 0
    L += w * l[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * __uint_as_float(ov[c][i] << 16);
      acc[2 * i + 1] += w * __uint_as_float(ov[c][i] & 0xffff0000u);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;  // no visible key: a zero output
  u32x4 pk;
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = f32x2_to_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
  *reinterpret_cast<u32x4*>(out + x_offset(a.out_qx, row, h * HD + r * 8, a.hq * HD)) = pk;
}

template <int HD>
hipError_t launch_prompt_hd(const AttnArgs& a, int nwq, hipStream_t st) {
  constexpr int QT = PROMPT_QT;
  const int Rall = a.R * (a.hq / a.hkv);
  dim3 grid((Rall + 16 * nwq * QT - 1) / (16 * nwq * QT), a.hkv, a.n_chunks > 1 ? a.n_chunks : 1);
  if (nwq == 4) hipLaunchKernelGGL((attn_prompt_kernel<HD, 4, QT>), grid, dim3(256), 0, st, a);
  else if (nwq == 2) hipLaunchKernelGGL((attn_prompt_kernel<HD, 2, QT>), grid, dim3(128), 0, st, a);
  else return hipErrorInvalidValue;
  if (a.n_chunks > 1 && a.n_chunks <= PROMPT_COMBINE_RANGES && !a.out_qx) {
    constexpr int VPB = 256 / (HD / 8);
    hipLaunchKernelGGL((attn_combine_few_kernel<HD>), dim3((Rall + VPB - 1) / VPB, a.hkv), dim3(256), 0,
                       st, a);
  } else if (a.n_chunks > 1) {
    dim3 cgrid(Rall, a.hkv, 1);
    hipLaunchKernelGGL((attn_combine_kernel<bf16_t, HD>), cgrid, dim3(WAVE), 0, st, a);
  }
  return hipGetLastError();
}

int attention_prompt_nwq(int R, int hq, int hkv) {
  // 4-wave workgroups (64 * QT query vectors sharing each K/V step) unless that leaves fewer
  // than 256 workgroups (a single KV head), then 2-wave ones
  return (R * (hq / hkv) + 64 * PROMPT_QT - 1) / (64 * PROMPT_QT) * hkv >= 256 ? 4 : 2;
}

int attention_prompt_block(int R, int hq, int hkv) {
  return 16 * PROMPT_QT * attention_prompt_nwq(R, hq, hkv);
}

hipError_t launch_attention_prompt(const AttnArgs& a, hipStream_t st) {
  if (a.B != 1 || a.vis != VIS_CAUSAL || a.R < 1 || a.hq % a.hkv) return hipErrorInvalidValue;
  if (a.n_chunks > 1 && (!a.part || a.chunk % 64 || a.n_launch != a.n_chunks)) return hipErrorInvalidValue;
  const int nwq = attention_prompt_nwq(a.R, a.hq, a.hkv);
  switch (a.hd) {
    case 64: return launch_prompt_hd<64>(a, nwq, st);
    case 128: return launch_prompt_hd<128>(a, nwq, st);
    case 256: return launch_prompt_hd<256>(a, nwq, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace specdec
