// Weight-streaming skinny GEMM: the kernel template and its launch dispatch.  Each
// (weight format, M-tile count) instantiation of dispatch_epi is compiled in a translation unit
// of its own (gemm_<format>_m<MT>.hip) so that the instantiations build in parallel; gemm.hip
// holds the entry point.
//
// Y[M][N] = X[M][Kd] . W[N][Kd]^T with W in the packed tile layout: each wave streams whole
// 1 KB tiles (bf16) with one 16-byte load per lane, so every weight byte is read from HBM
// exactly once per call and every wave load is fully contiguous.  The rows of X are padded to
// the 16-row MFMA tile; v_mfma_f32_16x16x32_bf16 (fp32: eight v_mfma_f32_16x16x4f32) does the
// contraction.  Weights may instead be in the 4-bit block format (one fp16 step per 32 weights):
// 1152-byte blocks of a 16-row tile and 128 reduction elements, one 16-byte code load per lane
// per block, expanded in registers to the same MFMA operand (q4_* below).
//
// Work split: a workgroup of NW waves owns UPW units (a unit = NU consecutive 16-row tiles, or a
// listed tile); the reduction axis of each unit is split over KW = NW / UPW waves, and the KW
// partial accumulators are summed through LDS in wave order.  KW depends only on (N, Kd), so a
// verify row and the same row in a decode step go through the same instruction sequence and
// come out bit-identical.  There is no communication between workgroups.
//
// RMSNorm without a pass of its own: rms(x) * w . W^T = s * ((x * w) . W^T) with the row scale
// s = 1/sqrt(mean(x^2) + eps).  The producer of the residual x also writes x * w_next in the
// storage type (w_next = the weight of the norm that reads x next) and per-16-column sums of
// squares of x; the consumer streams that operand like any other and multiplies its fp32
// results by s, formed in its epilogue from the sums of squares.  Epilogues: store / residual
// add, rotary embedding + KV-cache append, SiLU-gated product, per-unit argmax.

#pragma once

#include <math.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace specdec {
namespace gemm_detail {

// One lane's 16 (bf16) or 32 (fp32) bytes of a weight tile.  WC: weights that are read again
// soon and fit in the last-level cache (the drafter's, re-read every sub-step) use plain loads,
// which leave them cached; the target's weights, streamed once per step, use non-temporal loads
// (measured on MI355X: plain loads make the target's gate/up projection 11% slower and the
// drafter's sub-steps 9% faster).
template <typename T, bool WC>
__device__ __forceinline__ void load_w(Frag<T>& f, const T* W, size_t tile, int nkb, int kb,
                                       int lane) {
  const u32x4* p = reinterpret_cast<const u32x4*>(
      W + (tile * (size_t)nkb + (size_t)kb) * TILE_ELEMS + (size_t)lane * LANE_ELEMS);
  if constexpr (WC) {
    if constexpr (sizeof(T) == 2) {
      f.v = *p;
    } else {
      f.v[0] = p[0];
      f.v[1] = p[1];
    }
  } else if constexpr (sizeof(T) == 2) {
    f.v = __builtin_nontemporal_load(p);
  } else {
    f.v[0] = __builtin_nontemporal_load(p);
    f.v[1] = __builtin_nontemporal_load(p + 1);
  }
}

// Fragment of k-block J of a quad block q (X in the quad layout, one wave load per block): lane
// kg*16 + r takes lane kg*16 + 4J + r of its row of 16 (DPP row shift).  Lanes whose row is not
// 0..3 of k-block J feed only output rows >= 4, which no epilogue stores.
template <int J, typename T>
__device__ __forceinline__ void quad_frag(Frag<T>& f, const Frag<T>& q) {
  if constexpr (J == 0) {
    f = q;
  } else {
    constexpr int ctrl = 0x100 + 4 * J;  // row_shl:4J
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f.v[i] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)q.v[i], ctrl, 0xF, 0xF, true);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          f.v[h][i] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)q.v[h][i], ctrl, 0xF, 0xF, true);
    }
  }
}

template <typename T>
__device__ __forceinline__ void quad_frag_rt(Frag<T>& f, const Frag<T>& q, int j) {
  switch (j) {
    case 0: quad_frag<0>(f, q); break;
    case 1: quad_frag<1>(f, q); break;
    case 2: quad_frag<2>(f, q); break;
    default: quad_frag<3>(f, q); break;
  }
}


// ---- 4-bit block weights ----
// A lane's share of one (tile, k-group) block: 16 bytes of codes (four k-blocks of its 8
// elements) and the four fp16 steps of its row.  The code fragment of k-block j becomes the bf16
// MFMA operand 128 + code exactly (the code ORed into the mantissa of 128.0); a second product
// against the constant -136 gives the row sums of X times -136, which, fed in as the accumulator
// input, leaves X . (code - 8), and the k-block's step multiplies that in fp32.  The offset product
// depends only on X, so it is shared by every tile of the unit.
struct Q4Frag {
  u32x4 code;
  u32x2 step;
};

template <bool WC>
__device__ __forceinline__ void load_q4(Q4Frag& f, const uint8_t* W, size_t tile, int ngk, int g,
                                        int lane) {
  const uint8_t* blk = W + (tile * (size_t)ngk + (size_t)g) * Q4_BLOCK_BYTES;
  const u32x4* pc = reinterpret_cast<const u32x4*>(blk + lane * 16);
  const u32x2* ps = reinterpret_cast<const u32x2*>(blk + Q4_CODE_BYTES + (lane & 15) * 8);
  if constexpr (WC) {
    f.code = *pc;
    f.step = *ps;
  } else {
    f.code = __builtin_nontemporal_load(pc);
    f.step = __builtin_nontemporal_load(ps);
  }
}

// The two constants of the expansion, held in registers (made opaque once per kernel) so that
// each dword takes one v_and_or_b32 instead of an AND and an OR with literal operands.
struct Q4Consts {
  uint32_t mask, magic;
};
__device__ __forceinline__ Q4Consts q4_consts() {
  Q4Consts k{0x000F000Fu, 0x43004300u};
  asm volatile("" : "+s"(k.mask));
  asm volatile("" : "+v"(k.magic));
  return k;
}

__device__ __forceinline__ Frag<bf16_t> q4_operand(uint32_t c, const Q4Consts& k) {
  Frag<bf16_t> f;
  f.v = u32x4{(c & k.mask) | k.magic, ((c >> 4) & k.mask) | k.magic, ((c >> 8) & k.mask) | k.magic,
              ((c >> 12) & k.mask) | k.magic};
  return f;
}

__device__ __forceinline__ float q4_step(const Q4Frag& f, int j) {
  const uint32_t w = f.step[j >> 1];
  const uint16_t h = (j & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}

// X . (-136)^T: the accumulator input that turns X . (128 + code)^T into X . (code - 8)^T
__device__ __forceinline__ f32x4 q4_offset(const Frag<bf16_t>& xf) {
  Frag<bf16_t> m;
  m.v = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
  return mma<bf16_t>(xf, m, f32x4{0.f, 0.f, 0.f, 0.f});
}

// acc += d * t, elementwise (the k-block's product t scaled by its step d)
__device__ __forceinline__ void q4_scale_add(f32x4& acc, const f32x4& t, float d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(d, t[i], acc[i]);
}

// The main loops over the k-groups [g0, g1) for 4-bit block weights: X in the quad layout (at
// most 4 rows, one M-tile) or row-major (ML leading M-tiles).  The same ring of register stages
// as the bf16 loops; per k-block the operations are the same in both, so a row's result does not
// depend on the layout its call used.
template <int NU, bool WC>
__device__ __forceinline__ void q4_quad_loop(const GemmArgs& a, const size_t (&wt_tile)[NU], int g0,
                                             int g1, int lane, f32x4 (&acc)[NU][1]) {
  // k-groups per batch; two register stages (measured on MI355X at the 31B gate/up shape:
  // deeper rings and larger batches gain nothing)
  constexpr int GU = NU >= 2 ? 1 : 2;
  constexpr int S = 2;
  const uint8_t* W = reinterpret_cast<const uint8_t*>(a.W);
  const int ngk = a.nkb >> 2;
  const bf16_t* Xq = reinterpret_cast<const bf16_t*>(a.X) + (size_t)lane * 8;
  const Q4Consts kq = q4_consts();
  Q4Frag w[S][GU][NU];
  Frag<bf16_t> xq[S][GU];
  auto load_batch = [&](int st, int gb) {
#pragma unroll
    for (int gu = 0; gu < GU; ++gu) {
#pragma unroll
      for (int t = 0; t < NU; ++t) load_q4<WC>(w[st][gu][t], W, wt_tile[t], ngk, gb + gu, lane);
      load_frag<bf16_t>(xq[st][gu], Xq + (size_t)(gb + gu) * 512);
    }
  };
  auto mul_group = [&](const Q4Frag (&wg)[NU], const Frag<bf16_t>& q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Frag<bf16_t> xf;
      quad_frag_rt<bf16_t>(xf, q, j);
      const f32x4 off = q4_offset(xf);
#pragma unroll
      for (int t = 0; t < NU; ++t)
        q4_scale_add(acc[t][0], mma<bf16_t>(xf, q4_operand(wg[t].code[j], kq), off), q4_step(wg[t], j));
    }
  };
  const int nb = max(0, (g1 - g0) / GU);
  if (nb > 0) {
    auto g_of = [&](int i) { return g0 + min(i, nb - 1) * GU; };
#pragma unroll
    for (int st = 0; st < S - 1; ++st) load_batch(st, g_of(st));
    const int G = nb / S;
    for (int gi = 0; gi < G; ++gi) {
#pragma unroll
      for (int st = 0; st < S; ++st) {
        load_batch((st + S - 1) % S, g_of(gi * S + st + S - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gu = 0; gu < GU; ++gu) mul_group(w[st][gu], xq[st][gu]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int r = nb - G * S;
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < r) {
#pragma unroll
        for (int gu = 0; gu < GU; ++gu) mul_group(w[st][gu], xq[st][gu]);
      }
  }
  for (int g = g0 + nb * GU; g < g1; ++g) {
    Q4Frag wt[NU];
    Frag<bf16_t> q;
#pragma unroll
    for (int t = 0; t < NU; ++t) load_q4<WC>(wt[t], W, wt_tile[t], ngk, g, lane);
    load_frag<bf16_t>(q, Xq + (size_t)g * 512);
    mul_group(wt, q);
  }
}

template <int ML, int NU, int MT, bool WC>
__device__ __forceinline__ void q4_row_loop(const GemmArgs& a, const size_t (&wt_tile)[NU],
                                            const int (&xr)[MT], int g0, int g1, int lane,
                                            f32x4 (&acc)[NU][MT]) {
  constexpr int S = 2;
  const uint8_t* W = reinterpret_cast<const uint8_t*>(a.W);
  const int ngk = a.nkb >> 2;
  const bf16_t* Xb = reinterpret_cast<const bf16_t*>(a.X);
  const int kl = (lane >> 4) << 3;
  int xrow[ML];
  bool xok[ML];
#pragma unroll
  for (int mt = 0; mt < ML; ++mt) {
    xok[mt] = xr[mt] >= 0;
    xrow[mt] = xok[mt] ? xr[mt] : 0;
  }
  const Q4Consts kq = q4_consts();
  Q4Frag w[S][NU];
  Frag<bf16_t> x[S][4][ML];
  auto load_batch = [&](int st, int g) {
#pragma unroll
    for (int t = 0; t < NU; ++t) load_q4<WC>(w[st][t], W, wt_tile[t], ngk, g, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < ML; ++mt)
        load_frag<bf16_t>(x[st][j][mt], Xb + x_offset(a.x_qx, xrow[mt], (4 * g + j) * TILE_K + kl, a.ldx));
  };
  auto mul_group = [&](const Q4Frag (&wg)[NU], Frag<bf16_t> (&xg)[4][ML]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 off[ML];
#pragma unroll
      for (int mt = 0; mt < ML; ++mt) {
        if (!xok[mt]) zero_frag(xg[j][mt]);
        off[mt] = q4_offset(xg[j][mt]);
      }
#pragma unroll
      for (int t = 0; t < NU; ++t) {
        const Frag<bf16_t> wf = q4_operand(wg[t].code[j], kq);
        const float d = q4_step(wg[t], j);
#pragma unroll
        for (int mt = 0; mt < ML; ++mt)
          q4_scale_add(acc[t][mt], mma<bf16_t>(xg[j][mt], wf, off[mt]), d);
      }
    }
  };
  const int nb = max(0, g1 - g0);
  if (nb > 0) {
    auto g_of = [&](int i) { return g0 + min(i, nb - 1); };
    load_batch(0, g_of(0));
    const int G = nb / S;
    for (int gi = 0; gi < G; ++gi) {
#pragma unroll
      for (int st = 0; st < S; ++st) {
        load_batch((st + 1) % S, g_of(gi * S + st + 1));
        __builtin_amdgcn_sched_barrier(0);
        mul_group(w[st], x[st]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (nb - G * S > 0) mul_group(w[0], x[0]);
  }
}

// RMSNorm row scales 1/sqrt(sum_t yssq[t][r] / yscale_n + eps), from the sums of squares the
// producer of X left per 16-column tile t.  Every wave of a unit sums the tiles of its own
// reduction slice (tiles 2*kb0 .. 2*kb1, requested before its main loop): lane kg*16 + c adds
// tiles t0 + kg, t0 + kg + 4, ... of row c (+16 per M-tile) in ascending order, the four lane
// groups are added on the row swaps, and the unit's waves are added in wave order through LDS.
// The order is the same for every call size and layout, so a row's scale never depends on the
// call's other rows.
constexpr int RSL = 10;  // partials per lane and 16-row group requested ahead of the main loop
template <int MT> struct RowPart {
  float v[MT][RSL];
  int t0, t1;  // the wave's tile slice
};

// Local row of element v of M-tile mt in a lane.  The MFMA leaves rows (lane/16)*4 + v of
// column lane%16; with a single M-tile of at most 4 rows ("narrow") all rows sit in lanes 0-15,
// so the epilogue first moves row r to lanes 16r..16r+15 and then handles element 0 only, with
// every lane busy.  Elements that hold no row get an index past any M.
__device__ __forceinline__ int local_row(bool narrow, int mt, int v, int lane) {
  return narrow ? (v == 0 ? (lane >> 4) : (1 << 20)) : mt * 16 + ((lane >> 4) << 2) + v;
}

// Epilogue operands that do not depend on the products, read before the main loop so that their
// latency hides behind it: the norm weight and current value of each stored element (EPI_STORE),
// the rotary inverse frequency and the row positions (EPI_ROPE).
template <int MT, int NU> struct EpiPre {
  float wn[NU];
  float res[NU][MT][4];
  float2 cs[NU][MT][4];  // rotary (cos, sin) of the lane's pair at each row's position
  int pos[MT][4];        // rotary position of each row
};

template <int MT, int NU, int EPI>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& a, int tile0, int lane,
                                             EpiPre<MT, NU>& pre) {
  const int c16 = lane & 15;
  const bool narrow = MT == 1 && a.M <= 4;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int t = 0; t < NU; ++t) {
      const int col = min(tile0 + t, a.n_tiles - 1) * TILE_N + c16;
      pre.wn[t] = a.xw_out ? a.xw_norm[col] : 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = local_row(narrow, mt, v, lane);
          pre.res[t][mt][v] = (a.accumulate && m < a.M) ? a.out[(size_t)m * a.ldo + col] : 0.f;
        }
    }
  } else if constexpr (EPI == EPI_ROPE) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = local_row(narrow, mt, v, lane);
        const int b = m < a.M ? m / a.rows_per_seq : 0;
        const int r = m < a.M ? m - b * a.rows_per_seq : 0;  // row within its sequence
        pre.pos[mt][v] = a.len[b] + r + a.pos_off;
        // the other position rules (the mode is uniform over the launch): every row of a
        // sequence at len + pos_off, or a tree node at len + its depth (r < rows <= 64)
        if (a.pos_mode == POS_FLAT) pre.pos[mt][v] -= r;
        else if (a.pos_mode == POS_TREE) pre.pos[mt][v] += (int)a.tree_depth[r] - r - a.pos_off;
      }
    const int half = a.hd >> 1;
#pragma unroll
    for (int t = 0; t < NU; ++t) {
      const int col = min(tile0 + t, a.n_tiles - 1) * TILE_N + c16;
      const int i = (col % a.hd) >> 1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // a position outside the cache reads row 0 or the last (the epilogue flags it)
          const int pc = min(max(pre.pos[mt][v], 0), a.max_ctx - 1);
          pre.cs[t][mt][v] = a.rope_cs[(size_t)pc * half + i];
        }
    }
  }
}

__device__ __forceinline__ int yssq_ld(const GemmArgs& a) { return a.ld_yssq ? a.ld_yssq : a.M; }

template <int MT>
__device__ __forceinline__ void rowpart_load(const GemmArgs& a, int lane, int kb0, int kb1,
                                             RowPart<MT>& p) {
  p.t0 = min(2 * kb0, a.n_yssq);
  p.t1 = min(2 * kb1, a.n_yssq);
  const int ld = yssq_ld(a);
#pragma unroll
  for (int g = 0; g < MT; ++g) {
    const int row = min(g * 16 + (lane & 15), a.M - 1);
#pragma unroll
    for (int i = 0; i < RSL; ++i) {
      const int t = min(p.t0 + (lane >> 4) + 4 * i, a.n_yssq - 1);  // past the slice: not added
      p.v[g][i] = a.yssq[(size_t)t * ld + row];
    }
  }
}

// The wave's slice sums: part[g] for row g*16 + lane%16, identical in the four lanes of the row.
template <int MT>
__device__ __forceinline__ void rowpart_sum(const GemmArgs& a, int lane, const RowPart<MT>& p,
                                            float (&part)[MT]) {
  const int ld = yssq_ld(a);
#pragma unroll
  for (int g = 0; g < MT; ++g) {
    const int row = min(g * 16 + (lane & 15), a.M - 1);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RSL; ++i)
      if (p.t0 + (lane >> 4) + 4 * i < p.t1) s += p.v[g][i];
    // the slice's tiles past the prefetched ones, requested eight at a time and added in order
    int t = p.t0 + (lane >> 4) + 4 * RSL;
    for (; t + 28 < p.t1; t += 32) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = a.yssq[(size_t)(t + 4 * j) * ld + row];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; t < p.t1; t += 4) s += a.yssq[(size_t)t * ld + row];
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    part[g] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// The scale of each element of the lane's results, from `mine` = the scale of X row `lane`
// (r = the X row a local row reads: xr[mt] holds it for local row mt*16 + lane%16).
template <int MT>
__device__ __forceinline__ void row_scale_spread(const GemmArgs& a, int lane, const int (&xr)[MT],
                                                 float mine, float (&sc)[MT][4]) {
  const bool narrow = MT == 1 && a.M <= 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = __shfl(xr[mt], local_row(narrow, mt, v, lane) & 15, WAVE);
      sc[mt][v] = __shfl(mine, r < 0 ? 0 : (r & 63), WAVE);
    }
}

// ADDEND: compile the addend rows of EPI_STORE in (a launch that never has them leaves them out)
template <typename T, int MT, int NU, int EPI, bool ADDEND = true>
__device__ __forceinline__ void epilogue(const GemmArgs& a, f32x4 (&acc)[NU][MT], int u,
                                         int tile0, int grp, const int (&xr)[MT],
                                         float mine, const EpiPre<MT, NU>& pre, int lane) {
  const int c16 = lane & 15;
  const bool narrow = MT == 1 && a.M <= 4;
  if (narrow) {
    // row r of column c moves from element r of lane c to element 0 of lane 16r + c
    const int src = lane & 15, r = lane >> 4;
#pragma unroll
    for (int t = 0; t < NU; ++t) {
      const float x0 = __shfl(acc[t][0][0], src, WAVE), x1 = __shfl(acc[t][0][1], src, WAVE);
      const float x2 = __shfl(acc[t][0][2], src, WAVE), x3 = __shfl(acc[t][0][3], src, WAVE);
      acc[t][0][0] = r == 0 ? x0 : (r == 1 ? x1 : (r == 2 ? x2 : x3));
    }
  }
  if (a.yssq) {
    float sc[MT][4];
    row_scale_spread<MT>(a, lane, xr, mine, sc);
#pragma unroll
    for (int t = 0; t < NU; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][mt][v] *= sc[mt][v];
  }
  if constexpr (EPI == EPI_STORE) {
    // addend: a fixed-order sum of add_n row slices, read JB slices at a time for all of the
    // lane's elements (at most 16 values) so that the loads are in flight together
    constexpr int JB = 16 / (NU * MT * 4) > 1 ? 16 / (NU * MT * 4) : 1;
    float adds[NU][MT][4];
    const bool has_add = ADDEND && a.addend;
    if (has_add) {
#pragma unroll
      for (int t = 0; t < NU; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) adds[t][mt][v] = 0.f;
      for (int k0 = 0; k0 < a.add_n; k0 += JB) {
        float ld[JB][NU][MT][4];
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int t = 0; t < NU; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int m = min(local_row(narrow, mt, v, lane), a.M - 1);
                const int col = min(tile0 + t, a.n_tiles - 1) * TILE_N + c16;
                const int k = min(k0 + j, a.add_n - 1);
                ld[j][t][mt][v] = a.addend[((size_t)m * a.add_n + k) * a.ldo + col];
              }
#pragma unroll
        for (int j = 0; j < JB; ++j)
          if (k0 + j < a.add_n) {
#pragma unroll
            for (int t = 0; t < NU; ++t)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  adds[t][mt][v] = k0 + j == 0 ? ld[j][t][mt][v] : adds[t][mt][v] + ld[j][t][mt][v];
          }
      }
    }
#pragma unroll
    for (int t = 0; t < NU; ++t) {
      const int tile = tile0 + t;
      if (tile >= a.n_tiles) break;  // wave-uniform
      const int col = tile * TILE_N + c16;
      const float wn = pre.wn[t];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (narrow && v > 0) continue;  // uniform
          const int m = local_row(narrow, mt, v, lane);
          float sq = 0.f;
          if (m < a.M) {
            float* o = a.out + (size_t)m * a.ldo + col;
            float y = acc[t][mt][v];
            if (has_add) y = adds[t][mt][v] + y;
            if (a.accumulate) y = pre.res[t][mt][v] + y;
            *o = y;
            sq = y * y;
            if (a.xw_out)
              Elem<T>::store(reinterpret_cast<T*>(a.xw_out) + x_offset(a.out_qx, m, col, a.ldo), y * wn);
          }
          if (a.ssq) {
            const float r = sum16(sq);
            if (c16 == 0 && m < a.M) a.ssq[(size_t)tile * (a.ld_ssq ? a.ld_ssq : a.M) + m] = r;
          }
        }
    }
  } else if constexpr (EPI == EPI_ROPE) {
#pragma unroll
    for (int t = 0; t < NU; ++t) {
      const int tile = tile0 + t;
      if (tile >= a.n_tiles) break;  // wave-uniform
      const int col = tile * TILE_N + c16;
      const int hh = col / a.hd;
      const int p = col - hh * a.hd;
      const int i = p >> 1;
      const int second = p & 1;
      const int dim = i + second * (a.hd >> 1);
      const bool rot = hh < a.hq + a.hkv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (narrow && v > 0) continue;  // uniform
          const int m = local_row(narrow, mt, v, lane);
          const float val = acc[t][mt][v];
          const float partner = dpp_f32<DPP_XOR1>(val);  // the other element of the rotary pair
          if (m < a.M) {
            const int b = m / a.rows_per_seq;
            const int pos = pre.pos[mt][v];
            // cache slot: the position, except for a tree node (slot len + node index)
            const int slot = a.pos_mode == POS_TREE ? a.len[b] + (m - b * a.rows_per_seq) : pos;
            float y = val;
            if (rot) {
              const float cs = pre.cs[t][mt][v].x, sn = pre.cs[t][mt][v].y;
              const float x1 = second ? partner : val;
              const float x2 = second ? val : partner;
              y = second ? (x2 * cs + x1 * sn) : (x1 * cs - x2 * sn);
            }
            if (pos >= a.max_ctx || pos < 0) {
              // a query or key position outside the cache took a clamped rotary angle
              raise_error(a.err, ERRBIT_CAPACITY);
            }
            if (hh < a.hq) {
              Elem<T>::store(reinterpret_cast<T*>(a.qout) + ((size_t)m * a.hq + hh) * a.hd + dim, y);
            } else if (slot >= a.max_ctx || slot < 0) {
              raise_error(a.err, ERRBIT_CAPACITY);  // no cache slot: nothing is written
            } else {
              // K is stored [pos][hd], V transposed [hd][pos]
              const bool isk = hh < a.hq + a.hkv;
              const int g = isk ? hh - a.hq : hh - a.hq - a.hkv;
              T* cache = reinterpret_cast<T*>(isk ? a.kcache : a.vcache) + (size_t)b * a.cache_b_stride;
              const size_t off = isk ? ((size_t)g * a.max_ctx + slot) * a.hd + dim
                                     : ((size_t)g * a.hd + dim) * a.max_ctx + slot;
              Elem<T>::store(cache + off, y);
            }
          }
        }
    }
  } else if constexpr (EPI == EPI_SILU_G || EPI == EPI_STORE_G) {
    const int lt = tile0 - grp * a.tiles_per_group;  // tile within the group's matrix
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (narrow && v > 0) continue;  // uniform
        const int m = local_row(narrow, mt, v, lane);
        if (m >= a.M) continue;
        const int orow = a.orow_map[(size_t)grp * a.M + m];
        if (orow < 0) continue;
        if constexpr (EPI == EPI_SILU_G) {
          const float g = acc[0][mt][v];
          const float up = acc[1][mt][v];
          const float h = g / (1.0f + expf(-g)) * up;
          Elem<T>::store(reinterpret_cast<T*>(a.hout) + (size_t)orow * a.ldh + (lt >> 1) * TILE_N + c16, h);
        } else {
          a.out[(size_t)orow * a.ldo + lt * TILE_N + c16] =
              acc[0][mt][v] * a.orow_wt[(size_t)grp * a.M + m];
        }
      }
  } else if constexpr (EPI == EPI_SILU) {
    // tiles (2p, 2p+1) of the unit are the gate and up columns of product tile tile0/2 + p
#pragma unroll
    for (int p = 0; p < NU / 2; ++p) {
      if (tile0 + 2 * p >= a.n_tiles) break;  // wave-uniform
      const int f = ((tile0 >> 1) + p) * TILE_N + c16;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (narrow && v > 0) continue;  // uniform
          const int m = local_row(narrow, mt, v, lane);
          if (m < a.M) {
            const float g = acc[2 * p][mt][v];
            const float up = acc[2 * p + 1][mt][v];
            const float h = g / (1.0f + expf(-g)) * up;
            Elem<T>::store(reinterpret_cast<T*>(a.hout) + x_offset(a.out_qx, m, f, a.ldh), h);
          }
        }
    }
  } else {  // EPI_ARGMAX
    const int keep_row = a.unit_row ? a.unit_row[u] : -1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (narrow && v > 0) continue;  // uniform
        const int m = local_row(narrow, mt, v, lane);
        float best = -INFINITY;
        int bidx = 0x7fffffff;
        bool nan = false;
#pragma unroll
        for (int t = 0; t < NU; ++t) {
          const int tile = tile0 + t;
          if (tile < a.n_tiles) {
            const int col = tile * TILE_N + c16;
            const float y = acc[t][mt][v];
            nan |= (y != y);
            const int idx = a.idx_map ? a.idx_map[col] : col;
            argmax_combine(best, bidx, y, idx);
            // a listed unit belongs to one row: its other rows' products are not results
            if (a.logits && m < a.M && (keep_row < 0 || keep_row == m))
              a.logits[(size_t)m * a.ld_logits + col] = y;
          }
        }
        argmax16(best, bidx);
        if (nan && m < a.M) raise_error(a.err, ERRBIT_NAN);
        if (c16 == 0 && m < a.M && (keep_row < 0 || keep_row == m)) {
          // listed units belong to one row each and are stored by unit index
          const size_t slot = a.unit_row ? (size_t)u : (size_t)m * a.ld_amax + u;
          a.amax_val[slot] = best;
          a.amax_idx[slot] = bidx;
        }
      }
  }
}

// U: k-blocks per register stage (two stages are in flight) for NU = 1 / 2 / 4 tiles per unit;
// S: register stages of the quad-layout main loop (S - 1 batches in flight while one multiplies).
// Measured on MI355X at the 31B shapes: deeper rings gain nothing and cost occupancy.
constexpr int GEMM_U1 = 4, GEMM_U2 = 2, GEMM_U4 = 2;
constexpr int QSTAGES = 2;
template <int NU> struct QuadStages {
  static constexpr int S = QSTAGES;
};

template <int NU, int MT> struct Unroll {
  static constexpr int base = NU >= 4 ? GEMM_U4 : (NU == 2 ? GEMM_U2 : GEMM_U1);
  static constexpr int U = base / MT > 1 ? base / MT : 1;
};

template <typename T, int MT, int NU, int EPI, int NW, bool WC, bool Q4>
__global__ void __launch_bounds__(NW * 64) gemm_kernel(GemmArgs a) {
  __shared__ f32x4 red[NW * NU * 64];
  __shared__ float rsum[NW][64];  // per wave: its slice of each row's sum of squares
  const int lane = threadIdx.x & (WAVE - 1);
  // wave index, wave-uniform (readfirstlane tells the compiler, so the split bounds and the
  // main loop's trip count live in scalar registers and its branches are uniform)
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr bool GROUPED = EPI == EPI_SILU_G || EPI == EPI_STORE_G;
  const int KW = a.KW;
  const int ks = wid % KW;
  const int u = blockIdx.x * (NW / KW) + wid / KW;
  int n_units = a.n_units;
  if constexpr (GROUPED) n_units = min(n_units, a.n_groups_dev[0] * a.units_per_group);
  else if (a.n_units_dev) n_units = min(*a.n_units_dev, n_units);
  const bool active = u < n_units;
  int tile0 = 0, grp = 0;
  if (active) {
    if constexpr (GROUPED) {
      const int gi = u / a.units_per_group;
      grp = a.group_list[gi];
      tile0 = grp * a.tiles_per_group + (u - gi * a.units_per_group) * NU;
    } else {
      tile0 = a.unit_tile ? a.unit_tile[u] : u * NU;
    }
  }
  // X row read by local row mt*16 + lane%16 (-1: none)
  int xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    if constexpr (GROUPED) xr[mt] = (active && m < a.M) ? a.xrow_map[(size_t)grp * a.M + m] : -1;
    else xr[mt] = m < a.M ? m : -1;
  }
  const int kb0 = ks * a.kb_per_split;
  const int kb1 = min(a.nkb, kb0 + a.kb_per_split);
  const T* W = reinterpret_cast<const T*>(a.W);


  f32x4 acc[NU][MT];
#pragma unroll
  for (int t = 0; t < NU; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // epilogue operands and row-scale partials, requested before the main loop (the wave that
  // finishes each unit is the ks == 0 one)
  EpiPre<MT, NU> pre;
  if (active && ks == 0) epi_prefetch<MT, NU, EPI>(a, tile0, lane, pre);
  // this wave's share of the RMSNorm row-scale sums (all waves of the unit)
  const bool scaled = a.yssq != nullptr && active;  // wave-uniform
  RowPart<MT> rp;
  if (scaled) rowpart_load<MT>(a, lane, kb0, kb1, rp);

  if constexpr (Q4) {
    if (active) {
      size_t wt_tile[NU];
#pragma unroll
      for (int t = 0; t < NU; ++t) wt_tile[t] = (size_t)min(tile0 + t, a.n_tiles - 1);
      const int g0 = kb0 >> 2, g1 = kb1 >> 2;
      bool later_rows = false;  // does any M-tile after the first hold a row (wave-uniform)?
#pragma unroll
      for (int mt = 1; mt < MT; ++mt) later_rows |= __ballot(xr[mt] >= 0) != 0ull;
      if constexpr (MT == 1 && !GROUPED) {
        if (a.x_qx) q4_quad_loop<NU, WC>(a, wt_tile, g0, g1, lane, acc);
        else q4_row_loop<1, NU, MT, WC>(a, wt_tile, xr, g0, g1, lane, acc);
      } else if (MT == 1 || !later_rows) {
        q4_row_loop<1, NU, MT, WC>(a, wt_tile, xr, g0, g1, lane, acc);
      } else {
        q4_row_loop<MT, NU, MT, WC>(a, wt_tile, xr, g0, g1, lane, acc);
      }
    }
  }
  bool quad_done = Q4;
  if constexpr (MT == 1 && !Q4) {
    if (active && a.x_qx) {
      // X in the quad layout (at most 4 rows): one wave load per four k-blocks, shared by the
      // batch's k-blocks through DPP row shifts.  kb0 is a multiple of 4.
      // Loads are branch-free (a tile past n_tiles reads the last tile; its sums are never
      // stored), so the compiler's wait counts are exact and S - 1 batches stay in flight.
      constexpr int U = NU >= 4 ? 2 : 4;  // k-blocks per batch: a whole or half quad block
      constexpr int S = QuadStages<NU>::S;  // register stages, used as a ring
      Frag<T> w[S][U][NU];
      Frag<T> xq[S];
      int xl = lane;  // this lane's place in a quad block: row slot lane % 4
      if constexpr (GROUPED) {
        // a routed expert's rows are gathered: row slot r reads source row xrow_map[r] (a slot
        // no row was routed to reads row 0; its output row is never stored)
        const int src = __shfl(xr[0], lane & 3, WAVE);
        xl = lane - (lane & 3) + max(src, 0);
      }
      const T* Xq = reinterpret_cast<const T*>(a.X) + (size_t)xl * 8;
      size_t wt_tile[NU];
#pragma unroll
      for (int t = 0; t < NU; ++t) wt_tile[t] = (size_t)min(tile0 + t, a.n_tiles - 1);
      auto load_batch = [&](int st, int kbase) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
#pragma unroll
          for (int t = 0; t < NU; ++t) load_w<T, WC>(w[st][uu][t], W, wt_tile[t], a.nkb, kbase + uu, lane);
        load_frag<T>(xq[st], Xq + (size_t)(kbase >> 2) * 512);
      };
      auto mul_at = [&](auto j0c, int st) {
        constexpr int J0 = decltype(j0c)::value;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          Frag<T> xf;
          if constexpr (J0 + 0 == 0) {
            if (uu == 0) quad_frag<0>(xf, xq[st]);
            else if (uu == 1) quad_frag<1>(xf, xq[st]);
            else if (uu == 2) quad_frag<2>(xf, xq[st]);
            else quad_frag<3>(xf, xq[st]);
          } else {
            if (uu == 0) quad_frag<2>(xf, xq[st]);
            else quad_frag<3>(xf, xq[st]);
          }
#pragma unroll
          for (int t = 0; t < NU; ++t) acc[t][0] = mma<T>(xf, w[st][uu][t], acc[t][0]);
        }
      };
      auto mul_batch = [&](int st, int kbase) {
        if (U == 4 || (kbase & 2) == 0) mul_at(std::integral_constant<int, 0>{}, st);
        else mul_at(std::integral_constant<int, 2>{}, st);
      };
      const int nb = (kb1 - kb0) / U;
      if (nb > 0) {
        // Batch i of this wave sits in stage i % S.  Whole groups of S batches run in the loop,
        // each step prefetching S - 1 batches ahead (past the last batch it reads the last one
        // again; those stages are never multiplied); the r < S batches left over are already in
        // flight when the loop ends.  No step leaves the pipeline early, so every prefetch is
        // used on every path and stays where it is issued.
        auto kb_at = [&](int i) { return kb0 + i * U; };
        auto kb_of = [&](int i) { return kb_at(min(i, nb - 1)); };
#pragma unroll
        for (int st = 0; st < S - 1; ++st) load_batch(st, kb_of(st));
        const int G = nb / S;
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int st = 0; st < S; ++st) {
            // the prefetch is issued before this step's products wait for their stage
            load_batch((st + S - 1) % S, kb_of(g * S + st + S - 1));
            __builtin_amdgcn_sched_barrier(0);
            mul_batch(st, kb_at(g * S + st));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const int r = nb - G * S;
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
          if (st < r) mul_batch(st, kb_at(G * S + st));
      }
      for (int kb = kb0 + nb * U; kb < kb1; ++kb) {
        Frag<T> wt[NU], q, xf;
#pragma unroll
        for (int t = 0; t < NU; ++t) load_w<T, WC>(wt[t], W, wt_tile[t], a.nkb, kb, lane);
        load_frag<T>(q, Xq + (size_t)(kb >> 2) * 512);
        quad_frag_rt<T>(xf, q, kb & 3);
#pragma unroll
        for (int t = 0; t < NU; ++t) acc[t][0] = mma<T>(xf, wt[t], acc[t][0]);
      }
      quad_done = true;
    }
  }
  if constexpr (!Q4) if (active && !quad_done) {
    // Row-major X: the same ring of register stages as above.  Loads are branch-free: a tile past
    // the matrix reads the last one (its sums are never stored) and a row that does not exist reads
    // row 0, zeroed by a per-lane select before its product.  Only the leading M-tiles that hold a
    // row run (a routed expert gathers a few of the call's rows: its later M-tiles stay zero and
    // their rows are never stored).
    auto row_major = [&](auto mtc) {
      constexpr int ML = decltype(mtc)::value;
      constexpr int U = Unroll<NU, MT>::U;
      // register stages: one for the wide gated units (measured on MI355X at the 31B gate/up shape,
      // 32 rows: 122.5 -> 117.0 us; 139 registers and three waves per SIMD instead of 181 and two)
      constexpr int S = NU == 8 ? 1 : 2;
      Frag<T> w[S][U][NU];
      Frag<T> x[S][U][ML];
      size_t wt_tile[NU];
#pragma unroll
      for (int t = 0; t < NU; ++t) wt_tile[t] = (size_t)min(tile0 + t, a.n_tiles - 1);
      int xrow[ML];
      bool xok[ML];
#pragma unroll
      for (int mt = 0; mt < ML; ++mt) {
        xok[mt] = xr[mt] >= 0;
        xrow[mt] = xok[mt] ? xr[mt] : 0;
      }
      const T* Xb = reinterpret_cast<const T*>(a.X);
      const int kl = (lane >> 4) << 3;
      auto load_batch = [&](int st, int kbase) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
#pragma unroll
          for (int t = 0; t < NU; ++t) load_w<T, WC>(w[st][uu][t], W, wt_tile[t], a.nkb, kbase + uu, lane);
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
#pragma unroll
          for (int mt = 0; mt < ML; ++mt)
            load_frag<T>(x[st][uu][mt], Xb + x_offset(a.x_qx, xrow[mt], (kbase + uu) * TILE_K + kl, a.ldx));
      };
      auto mul_batch = [&](int st) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu)
#pragma unroll
          for (int mt = 0; mt < ML; ++mt) {
            Frag<T> xf = x[st][uu][mt];
            if (!xok[mt]) zero_frag(xf);
#pragma unroll
            for (int t = 0; t < NU; ++t) acc[t][mt] = mma<T>(xf, w[st][uu][t], acc[t][mt]);
          }
      };
      const int nb = (kb1 - kb0) / U;  // whole batches
      if (nb > 0) {
        auto kb_of = [&](int i) { return kb0 + min(i, nb - 1) * U; };
#pragma unroll
        for (int st = 0; st < S - 1; ++st) load_batch(st, kb_of(st));
        const int G = nb / S;
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int st = 0; st < S; ++st) {
            load_batch((st + S - 1) % S, kb_of(g * S + st + S - 1));
            __builtin_amdgcn_sched_barrier(0);
            mul_batch(st);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const int r = nb - G * S;
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
          if (st < r) mul_batch(st);
      }
      for (int kb = kb0 + nb * U; kb < kb1; ++kb) {
        Frag<T> wt[NU];
        Frag<T> xt[ML];
#pragma unroll
        for (int t = 0; t < NU; ++t) load_w<T, WC>(wt[t], W, wt_tile[t], a.nkb, kb, lane);
#pragma unroll
        for (int mt = 0; mt < ML; ++mt) {
          load_frag<T>(xt[mt], Xb + x_offset(a.x_qx, xrow[mt], kb * TILE_K + kl, a.ldx));
          if (!xok[mt]) zero_frag(xt[mt]);
        }
#pragma unroll
        for (int t = 0; t < NU; ++t)
#pragma unroll
          for (int mt = 0; mt < ML; ++mt) acc[t][mt] = mma<T>(xt[mt], wt[t], acc[t][mt]);
      }
    };
    bool later_rows = false;  // does any M-tile after the first hold a row (wave-uniform)?
#pragma unroll
    for (int mt = 1; mt < MT; ++mt) later_rows |= __ballot(xr[mt] >= 0) != 0ull;
    if (MT == 1 || !later_rows) row_major(std::integral_constant<int, 1>{});
    else row_major(std::integral_constant<int, MT>{});
  }

  float part[MT];
  if (scaled) rowpart_sum<MT>(a, lane, rp, part);
  float mine = 1.f;  // the RMSNorm scale of X row `lane`
  auto finish_scale = [&](float total) { mine = 1.0f / sqrtf(total / (float)a.yscale_n + a.eps); };
  if (KW > 1) {
    // the row-scale slices of the unit's waves, added in wave order after the first barrier
    if (scaled && lane < 16) {
#pragma unroll
      for (int g = 0; g < MT; ++g) rsum[wid][g * 16 + lane] = part[g];
    }
    // sum the KW partial accumulators of each unit in wave order, one M-tile at a time
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (ks != 0) {
#pragma unroll
        for (int t = 0; t < NU; ++t) red[(wid * NU + t) * 64 + lane] = acc[t][mt];
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int t = 0; t < NU; ++t) {
          f32x4 s = acc[t][mt];
          for (int k2 = 1; k2 < KW; ++k2) s += red[((wid + k2) * NU + t) * 64 + lane];
          acc[t][mt] = s;
        }
      }
      __syncthreads();
    }
    if (ks != 0) return;
    if (scaled) {
      float total = rsum[wid][lane];
      for (int k2 = 1; k2 < KW; ++k2) total += rsum[wid + k2][lane];
      finish_scale(total);
    }
  } else if (scaled) {
    // one wave: every lane of column c holds the sums of rows g*16 + c, so lane `lane` has row
    // `lane` in part[lane / 16]
    float total = part[0];
#pragma unroll
    for (int g = 1; g < MT; ++g)
      if ((lane >> 4) == g) total = part[g];
    finish_scale(total);
  }
  if (!active) return;
  epilogue<T, MT, NU, EPI>(a, acc, u, tile0, grp, xr, mine, pre, lane);
}

template <typename T, int MT, int NU, int EPI, int NW, bool WC, bool Q4>
hipError_t launch_wc(const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  const int upw = NW / a.KW;
  dim3 grid((a.n_units + upw - 1) / upw), block(NW * 64);
  if (tm)
    hipExtLaunchKernelGGL((gemm_kernel<T, MT, NU, EPI, NW, WC, Q4>), grid, block, 0, st, tm->start,
                          tm->stop, 0, a);
  else
    hipLaunchKernelGGL((gemm_kernel<T, MT, NU, EPI, NW, WC, Q4>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename T, int MT, int NU, int EPI, int NW, bool Q4>
hipError_t launch_t(const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  return a.w_cached ? launch_wc<T, MT, NU, EPI, NW, true, Q4>(a, st, tm)
                    : launch_wc<T, MT, NU, EPI, NW, false, Q4>(a, st, tm);
}

template <typename T, int MT, int NU, int EPI, bool Q4>
hipError_t launch_nw(const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  if constexpr (NU < 4) {
    if (a.NW == 16) return launch_t<T, MT, NU, EPI, 16, Q4>(a, st, tm);
  }
  if (a.NW == 8) return launch_t<T, MT, NU, EPI, 8, Q4>(a, st, tm);
  if (a.NW == 4) return launch_t<T, MT, NU, EPI, 4, Q4>(a, st, tm);
  return hipErrorInvalidValue;
}

// Q4: 4-bit block weights (bf16 activations only)
template <typename T, int MT, bool Q4>
hipError_t dispatch_epi(int NU, int epi, const GemmArgs& a, hipStream_t st,
                       const LaunchTiming* tm) {
  if (epi == EPI_STORE && NU == 1) return launch_nw<T, MT, 1, EPI_STORE, Q4>(a, st, tm);
  if (epi == EPI_STORE && NU == 2) return launch_nw<T, MT, 2, EPI_STORE, Q4>(a, st, tm);
  if (epi == EPI_ROPE && NU == 1) return launch_nw<T, MT, 1, EPI_ROPE, Q4>(a, st, tm);
  if (epi == EPI_ROPE && NU == 2) return launch_nw<T, MT, 2, EPI_ROPE, Q4>(a, st, tm);
  if (epi == EPI_SILU && NU == 2) return launch_nw<T, MT, 2, EPI_SILU, Q4>(a, st, tm);
  // gated units of four gate/up pairs: bf16 calls of 17..32 rows
  if constexpr (MT == 2 && !Q4 && sizeof(T) == 2) {
    if (epi == EPI_SILU && NU == 8) return launch_nw<T, MT, 8, EPI_SILU, Q4>(a, st, tm);
    if (epi == EPI_SILU && NU == 4) return launch_nw<T, MT, 4, EPI_SILU, Q4>(a, st, tm);
  }
  if (epi == EPI_SILU_G && NU == 2) return launch_nw<T, MT, 2, EPI_SILU_G, Q4>(a, st, tm);
  if (epi == EPI_STORE_G && NU == 1) return launch_nw<T, MT, 1, EPI_STORE_G, Q4>(a, st, tm);
  if (epi == EPI_ARGMAX && NU == 4) return launch_nw<T, MT, 4, EPI_ARGMAX, Q4>(a, st, tm);
  return hipErrorInvalidValue;
}

template <typename T, bool Q4>
hipError_t dispatch_mt(int MT, int NU, int epi, const GemmArgs& a, hipStream_t st,
                       const LaunchTiming* tm) {
  switch (MT) {
    case 1: return dispatch_epi<T, 1, Q4>(NU, epi, a, st, tm);
    case 2: return dispatch_epi<T, 2, Q4>(NU, epi, a, st, tm);
    case 4: return dispatch_epi<T, 4, Q4>(NU, epi, a, st, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm_detail
}  // namespace specdec
