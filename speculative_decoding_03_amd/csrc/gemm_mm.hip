// Compute-bound GEMM for prompt chunks (prefill): Y[M][N] = X[M][Kd] . W[N][Kd]^T with M in the
// hundreds, where every weight byte feeds M rows and the MFMA units, not HBM, set the pace.
//
// A workgroup of WM x WN waves computes a block of 64*WM rows x 64*WN columns; wave (wm, wn) owns
// the 64 x 64 sub-block of four 16-row M-tiles and four 16-column tiles, held as the same
// accumulator array the skinny kernel uses (acc[tile][M-tile]), so the skinny kernel's epilogues
// (residual add + sums of squares + x * w_next, rotary + KV append, SiLU product, per-unit argmax)
// apply unchanged to each wave's sub-block.  The reduction axis streams in stages of two k-blocks
// (64 elements): every thread copies 16-byte runs of X rows and of packed weight tiles from
// global memory into LDS, laid out in MFMA operand order (a fragment = 64 lanes x 16 bytes,
// contiguous), so each wave reads its four X fragments and four weight fragments per k-block
// with conflict-free 16-byte LDS reads and issues sixteen v_mfma_f32_16x16x32_bf16.  Two LDS
// stages alternate: the next D stages' global loads are in flight (a register ring) while the
// current one is multiplied, and one barrier per stage separates writing a stage from reading it.
// Wide projections take 256 x 256 blocks (16 waves), narrower ones 128 x 128 or 64 x 128.  The
// per-row, per-tile reduction order is fixed (k-blocks ascending), independent of M and of the
// block shape.

#include "gemm_impl.h"

namespace specdec {
namespace gemm_detail {

template <int EPI>
__device__ void mm_finish(const GemmArgs& a, f32x4 (&acc)[4][4], int m0, int tile0, int lane);
__device__ void mm_rope_store(const GemmArgs& a, f32x4 (&acc)[4][4], int m0, int tile0, int lane,
                              bool act, uint16_t* lds);

// The RMSNorm scale 1/sqrt(sum_t yssq[t][m] / yscale_n + eps) of row m = m0 + lane: the row's
// per-tile partials (contiguous across the lanes for each t) are added into RS running sums, sum
// j taking tiles j, j + RS, ..., with RS loads in flight at a time, and the sums added in j order.
__device__ __forceinline__ float prompt_row_scale(const GemmArgs& a, int m0, int lane) {
  constexpr int RS = 16;
  const int m = min(m0 + lane, a.M - 1);
  const float* y = a.yssq + m;
  float s[RS];
#pragma unroll
  for (int j = 0; j < RS; ++j) s[j] = 0.f;
  int t = 0;
  for (; t + RS <= a.n_yssq; t += RS) {
    float v[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) v[j] = y[(size_t)(t + j) * a.M];
#pragma unroll
    for (int j = 0; j < RS; ++j) s[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < RS; ++j)
    if (t + j < a.n_yssq) s[j] += y[(size_t)(t + j) * a.M];
  float ss = s[0];
#pragma unroll
  for (int j = 1; j < RS; ++j) ss += s[j];
  return 1.0f / sqrtf(ss / (float)a.yscale_n + a.eps);
}

// The partial block of split z (k-range z of kpart_n) in MFMA accumulator order: wave w of block
// (bx, by) holds 16 fragments (tile, M-tile) of 64 lanes x 4 floats, each a contiguous 1 KB.
// Offset in floats of the wave's 16 x 64 x 4 floats.
__device__ __forceinline__ size_t mm_part_offset(int z, int nblk, int blk, int nw, int w) {
  return (((size_t)z * nblk + blk) * nw + w) * (16 * 64 * 4);
}

// One lane's weight fragment (8 consecutive k of one row) of a 4-bit block matrix as bf16: the
// lane's code word c (element e at bit (e % 2) * 16 + (e / 2) * 4) and the block's fp16 step h;
// each weight d * (q - 8) is exact in fp32 and rounded to bf16 (nearest even) for the MFMA.
__device__ __forceinline__ u32x4 q4_fragment_bf16(uint32_t c, uint32_t h) {
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  const float o = -8.0f * d;
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;  // bytes e0 e4 e1 e5 / e2 e6 e3 e7
  auto w = [&](uint32_t x, int byte) { return __builtin_fmaf(d, (float)((x >> (8 * byte)) & 0xFFu), o); };
  return u32x4{f32x2_to_bf16x2(w(lo, 0), w(lo, 2)), f32x2_to_bf16x2(w(hi, 0), w(hi, 2)),
               f32x2_to_bf16x2(w(lo, 1), w(lo, 3)), f32x2_to_bf16x2(w(hi, 1), w(hi, 3))};
}

template <int EPI, int WM, int WN, int KS, int D, bool SPLIT, bool Q4W = false>
__global__ void __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4 > 2 ? WM * WN / 4 : 2))) mm_kernel(GemmArgs a) {
  constexpr int MM_KS = KS;               // k-blocks per LDS stage
  constexpr int NTH = WM * WN * 64;
  constexpr int BMT = 4 * WM;             // 16-row M-tiles per block
  constexpr int BNT = 4 * WN;             // 16-column tiles per block
  constexpr int A_FR = MM_KS * BMT;       // X fragments per stage
  constexpr int B_FR = MM_KS * BNT;       // weight fragments per stage
  constexpr int A_RUNS = A_FR * 64 / NTH;  // 16-byte runs each thread copies per stage
  constexpr int B_RUNS = B_FR * 64 / NTH;
  static_assert(A_FR * 64 % NTH == 0 && B_FR * 64 % NTH == 0, "stage does not split evenly");
  __shared__ __align__(16) u32x4 sa[2][A_FR * 64];
  __shared__ __align__(16) u32x4 sb[2][B_FR * 64];

  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % WM, wn = w / WM;
  const int m_blk = blockIdx.y * 64 * WM, t_blk = blockIdx.x * BNT;
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.X);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.W);
  const int nkb = a.nkb;
  // stages [st0, st0 + n_st) of the reduction: all of it, or split blockIdx.z of kpart_n
  int st0 = 0, n_st = nkb / MM_KS;
  if constexpr (SPLIT) {
    const int z = blockIdx.z, tot = n_st;
    st0 = (int)((long)tot * z / a.kpart_n);
    n_st = (int)((long)tot * (z + 1) / a.kpart_n) - st0;
  }

  // this thread's runs: run i = tid + j*NTH is lane i % 64 of fragment i / 64, so a wave writes
  // one whole fragment (64 consecutive 16-byte LDS slots, no bank conflict).  X fragment f is
  // M-tile f % BMT at k-block f / BMT: lane kg*16 + r holds row r, elements kg*8 .. kg*8+7;
  // weight fragment f is block tile f / KS at k-block f % KS.  Rows past M and tiles past N read
  // the last row / tile (their results are never stored).
  const bf16_t* xsrc[A_RUNS];
  int adst[A_RUNS];
#pragma unroll
  for (int j = 0; j < A_RUNS; ++j) {
    const int i = tid + j * NTH;
    const int fr = i / 64, ln = i % 64;
    const int kb = fr / BMT, mt = fr % BMT;
    const int row = mt * 16 + (ln & 15);
    xsrc[j] = X + (size_t)min(m_blk + row, a.M - 1) * a.ldx + kb * TILE_K + (ln >> 4) * 8;
    adst[j] = fr * 64 + ln;
  }
  const bf16_t* wsrc[B_RUNS];
  const uint8_t* qsrc[B_RUNS];  // 4-bit weights: the run's code word in its tile's first block
  int bdst[B_RUNS];
#pragma unroll
  for (int j = 0; j < B_RUNS; ++j) {
    const int i = tid + j * NTH;
    const int fr = i / 64, ln = i % 64;
    const int kb = fr % MM_KS, t = fr / MM_KS;
    const size_t tt = (size_t)min(t_blk + t, a.n_tiles - 1);
    if constexpr (Q4W) {
      qsrc[j] = reinterpret_cast<const uint8_t*>(a.W) + tt * (size_t)(nkb >> 2) * Q4_BLOCK_BYTES + ln * 16;
      wsrc[j] = nullptr;
    } else {
      wsrc[j] = W + (tt * nkb + kb) * TILE_ELEMS + ln * LANE_ELEMS;
      qsrc[j] = nullptr;
    }
    bdst[j] = (kb * BNT + t) * 64 + ln;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // D stages in flight in a register ring (slot = stage % D); a stage past the last one reads the
  // last one again and is never stored
  u32x4 ra[D][A_RUNS], rb[D][Q4W ? 1 : B_RUNS];
  uint32_t rq[D][Q4W ? B_RUNS : 1], rh[D][Q4W ? B_RUNS : 1];  // 4-bit: code word and step
  auto load_stage = [&](int slot, int st) {
    const int s = st0 + min(st, n_st - 1);
#pragma unroll
    for (int j = 0; j < A_RUNS; ++j) ra[slot][j] = *reinterpret_cast<const u32x4*>(xsrc[j] + s * MM_KS * TILE_K);
#pragma unroll
    for (int j = 0; j < B_RUNS; ++j) {
      if constexpr (Q4W) {
        // k-block kbg of the stage: word kbg % 4 of the lane's 16 bytes in block kbg / 4, and
        // the step of the lane's row there
        const int i = tid + j * NTH, ln = i % 64;
        const int kbg = s * MM_KS + (i / 64) % MM_KS;
        const uint8_t* blk = qsrc[j] - ln * 16 + (size_t)(kbg >> 2) * Q4_BLOCK_BYTES;
        rq[slot][j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(blk + ln * 16 + (kbg & 3) * 4));
        rh[slot][j] = *reinterpret_cast<const uint16_t*>(blk + Q4_CODE_BYTES + (ln & 15) * 8 + (kbg & 3) * 2);
      } else {
        rb[slot][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[j] + (size_t)s * MM_KS * TILE_ELEMS));
      }
    }
  };
  auto store_stage = [&](int slot, int buf) {
#pragma unroll
    for (int j = 0; j < A_RUNS; ++j) sa[buf][adst[j]] = ra[slot][j];
#pragma unroll
    for (int j = 0; j < B_RUNS; ++j) {
      if constexpr (Q4W) sb[buf][bdst[j]] = q4_fragment_bf16(rq[slot][j], rh[slot][j]);
      else sb[buf][bdst[j]] = rb[slot][j];
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kb = 0; kb < MM_KS; ++kb) {
      Frag<bf16_t> xf[4], wf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xf[mt].v = sa[buf][(kb * BMT + wm * 4 + mt) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) wf[t].v = sb[buf][(kb * BNT + wn * 4 + t) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[t][mt] = mma<bf16_t>(xf[mt], wf[t], acc[t][mt]);
    }
  };

  if (n_st > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_stage(d, d);
    // Stage s: copied from its register slot into LDS buffer s % 2 (last read by stage s - 2,
    // which every wave finished before the previous barrier), its slot refilled with stage
    // s + D, one barrier, then multiplied.
    for (int s0 = 0; s0 < n_st; s0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        if (s < n_st) {  // uniform
          store_stage(d, s & 1);
          load_stage(d, s + D);
          __syncthreads();
          compute(s & 1);
        }
      }
    }
  }

  if constexpr (SPLIT) {
    // this split's sums, for the reduction launch
    float* dst = a.kpart + mm_part_offset(blockIdx.z, gridDim.x * gridDim.y,
                                          blockIdx.y * gridDim.x + blockIdx.x, WM * WN, w);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<f32x4*>(dst + ((t * 4 + mt) * 64 + lane) * 4) = acc[t][mt];
    return;
  }
  if constexpr (EPI == EPI_ROPE && WM * WN <= 4) {
    // every wave is done with the stage buffers; each takes 8 KB of the weight buffers for its
    // sub-block's outputs (two more barriers inside, reached by every wave)
    static_assert(sizeof(sb) >= (size_t)WM * WN * 64 * 64 * 2, "LDS for the rotary outputs");
    __syncthreads();
    const int m0 = m_blk + wm * 64, tile0 = t_blk + wn * 4;
    mm_rope_store(a, acc, m0, tile0, lane, m0 < a.M && tile0 < a.n_tiles,
                  reinterpret_cast<uint16_t*>(&sb[0][0]) + w * 64 * 64);
    return;
  }
  mm_finish<EPI>(a, acc, m_blk + wm * 64, t_blk + wn * 4, lane);
}

// Sums the kpart_n partial blocks of a split prompt GEMM in split order, then applies the
// epilogue.  Workgroups of 4 waves (the epilogue's registers); block (x, y) of the split launch
// is covered by workgroups (x, y, 0 .. WM*WN/4 - 1), wave w of the block by workgroup w / 4.
template <int EPI, int WM, int WN>
__global__ void __launch_bounds__(256) mm_reduce_kernel(GemmArgs a) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.z * 4 + (threadIdx.x >> 6));
  const int wm = w % WM, wn = w / WM;
  const int nblk = gridDim.x * gridDim.y, blk = blockIdx.y * gridDim.x + blockIdx.x;
  f32x4 acc[4][4];
  for (int z = 0; z < a.kpart_n; ++z) {
    const float* src = a.kpart + mm_part_offset(z, nblk, blk, WM * WN, w);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + ((t * 4 + mt) * 64 + lane) * 4);
        acc[t][mt] = z == 0 ? v : acc[t][mt] + v;
      }
  }
  const int m0 = blockIdx.y * 64 * WM + wm * 64, tile0 = blockIdx.x * 4 * WN + wn * 4;
  if constexpr (EPI == EPI_ROPE) {
    __shared__ __align__(16) uint16_t rl[4][64 * 64];  // each wave's rotary outputs
    mm_rope_store(a, acc, m0, tile0, lane, m0 < a.M && tile0 < a.n_tiles, rl[threadIdx.x >> 6]);
    return;
  }
  mm_finish<EPI>(a, acc, m0, tile0, lane);
}

// ---- the skinny kernel's epilogue on one wave's 64 x 64 sub-block (rows m0.., tiles tile0..) ----
template <int EPI>
__device__ void mm_finish(const GemmArgs& a, f32x4 (&acc)[4][4], int m0, int tile0, int lane) {
  if (m0 >= a.M || tile0 >= a.n_tiles) return;
  GemmArgs e = a;
  e.M = min(64, a.M - m0);
  e.x_qx = e.out_qx = 0;
  if (a.yssq) {
    // RMSNorm row scales of the 64 rows, one row per lane (prompt_row_scale)
    const float mine = prompt_row_scale(a, m0, lane);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sc = __shfl(mine, mt * 16 + ((lane >> 4) << 2) + v, WAVE);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][mt][v] *= sc;
      }
    e.yssq = nullptr;
  }
  if constexpr (EPI == EPI_STORE) {
    e.out = a.out + (size_t)m0 * a.ldo;
    e.ld_ssq = a.M;
    if (e.ssq) e.ssq = a.ssq + m0;
    if (e.xw_out) e.xw_out = reinterpret_cast<bf16_t*>(a.xw_out) + (size_t)m0 * a.ldo;
  } else if constexpr (EPI == EPI_ROPE) {
    e.qout = reinterpret_cast<bf16_t*>(a.qout) + (size_t)m0 * a.hq * a.hd;
    e.rows_per_seq = 1 << 30;  // one sequence
    e.pos_off = a.pos_off + m0;
  } else if constexpr (EPI == EPI_SILU) {
    e.hout = reinterpret_cast<bf16_t*>(a.hout) + (size_t)m0 * a.ldh;
  } else {
    e.amax_val = a.amax_val + (size_t)m0 * a.ld_amax;
    e.amax_idx = a.amax_idx + (size_t)m0 * a.ld_amax;
    if (e.logits) e.logits = a.logits + (size_t)m0 * a.ld_logits;
    e.unit_row = nullptr;
  }
  int xr[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = mt * 16 + (lane & 15);
    xr[mt] = m < e.M ? m : -1;
  }
  if constexpr (EPI == EPI_ARGMAX) {
    // one argmax unit of 64 columns
    EpiPre<4, 4> pre;
    epilogue<bf16_t, 4, 4, EPI, false>(e, acc, tile0 >> 2, tile0, 0, xr, 1.f, pre, lane);
  } else {
    // two halves of two tiles each (for SiLU: a gate and an up tile), so that the epilogue's
    // prefetched operands stay within the main loop's register budget
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int t0 = tile0 + 2 * hh;
      if (t0 >= e.n_tiles) break;  // uniform
      f32x4 (&part)[2][4] = *reinterpret_cast<f32x4 (*)[2][4]>(&acc[2 * hh][0]);
      EpiPre<4, 2> pre;
      epi_prefetch<4, 2, EPI>(e, t0, lane, pre);
      epilogue<bf16_t, 4, 2, EPI, false>(e, part, t0 >> 1, t0, 0, xr, 1.f, pre, lane);
      __builtin_amdgcn_sched_barrier(0);  // the halves' registers do not overlap
    }
  }
}

// ---- q/k/v + RoPE + K/V append of one wave's 64 x 64 sub-block of a prompt chunk (rows m0.., tiles
// tile0 .. tile0 + 3: 64 columns of one head, as heads are multiples of 64 columns; one sequence,
// positions len[0] + pos_off + row).  The rotated values go to the wave's 8 KB of LDS in output
// order, then out as contiguous runs: q and K rows ([row][hd], [pos][hd]) 16 bytes per lane, each
// V^T row ([hd][pos]) 64 consecutive positions per instruction (the chunk's first position has any
// alignment).  The rotary pairs are adjacent columns (2i, 2i + 1) and land at dims i and
// i + hd / 2, as in the skinny kernel's epilogue.  Every wave of the workgroup calls this (one
// barrier inside); `act`: the sub-block holds rows and columns.  A row whose position falls
// outside the cache raises the capacity bit and its K and V are not written.  LDS element (r, j) of a 64 x 64
// array sits at r * 64 + ((j / 8) ^ (r % 8)) * 8 + j % 8, so that neither the column writes nor
// the row reads meet in a bank. ----
__device__ __forceinline__ int rope_lds(int r, int j) { return r * 64 + ((((j >> 3) ^ r) & 7) << 3) + (j & 7); }

__device__ void mm_rope_store(const GemmArgs& a, f32x4 (&acc)[4][4], int m0, int tile0, int lane,
                              bool act, uint16_t* lds) {
  const int c16 = lane & 15, grp = lane >> 4;
  const int hd = a.hd, half = hd >> 1;
  const int col0 = tile0 * TILE_N;
  const int hh = col0 / hd, p0 = col0 - hh * hd;  // head, and its first column here (even)
  const bool isq = hh < a.hq, isk = !isq && hh < a.hq + a.hkv;
  const int rows = min(64, a.M - m0);
  const int pos0 = act ? a.len[0] + a.pos_off + m0 : 0;  // position of row m0
  const bool in_cache = pos0 >= 0 && pos0 + rows <= a.max_ctx;
  if (act) {
    if (a.yssq) {
      // RMSNorm row scales of the 64 rows, one row per lane
      const float mine = prompt_row_scale(a, m0, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float sc = __shfl(mine, mt * 16 + (grp << 2) + v, WAVE);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t][mt][v] *= sc;
        }
    }
    // a position outside the cache takes a clamped rotary angle: flagged, and its row's K and V are
    // not written
    if (!in_cache && lane == 0) raise_error(a.err, ERRBIT_CAPACITY);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = t * 16 + c16;                     // column within the sub-block
      const int j = (c & 1) * 32 + (c >> 1);          // its dim among the sub-block's 64
      const int ip = (p0 + c) >> 1;                   // rotary pair index
      float2 cs[4][4];
      if (isq || isk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int pc = min(max(pos0 + mt * 16 + (grp << 2) + v, 0), a.max_ctx - 1);
            cs[mt][v] = a.rope_cs[(size_t)pc * half + ip];
          }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = mt * 16 + (grp << 2) + v;
          const float val = acc[t][mt][v];
          const float partner = dpp_f32<DPP_XOR1>(val);
          float y = val;
          if (isq || isk) {
            const bool second = c & 1;
            const float x1 = second ? partner : val, x2 = second ? val : partner;
            y = second ? (x2 * cs[mt][v].x + x1 * cs[mt][v].y) : (x1 * cs[mt][v].x - x2 * cs[mt][v].y);
          }
          lds[isq || isk ? rope_lds(r, j) : rope_lds(j, r)] = f32_to_bf16(y);
        }
    }
  }
  __syncthreads();
  if (!act) return;
  auto slot_ok = [&](int r) { return isq || (pos0 + r >= 0 && pos0 + r < a.max_ctx); };
  if (isq || isk) {
    // 64 rows x 8 runs of 8 dims, one 16-byte run per lane at a time
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int sidx = jj * 64 + lane, r = sidx >> 3, q = sidx & 7;
      if (r >= rows || !slot_ok(r)) continue;
      const int d0 = (q >> 2) * half + (p0 >> 1) + (q & 3) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + rope_lds(r, q * 8));
      bf16_t* dst = isq ? reinterpret_cast<bf16_t*>(a.qout) + ((size_t)(m0 + r) * a.hq + hh) * hd + d0
                        : reinterpret_cast<bf16_t*>(a.kcache) +
                              ((size_t)(hh - a.hq) * a.max_ctx + pos0 + r) * hd + d0;
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  } else {
    const int g = hh - a.hq - a.hkv;
    uint16_t* vt = reinterpret_cast<uint16_t*>(a.vcache);
    for (int j = 0; j < 64; ++j) {
      const int dim = (j >> 5) * half + (p0 >> 1) + (j & 31);
      if (lane < rows && slot_ok(lane)) vt[((size_t)g * hd + dim) * a.max_ctx + pos0 + lane] = lds[rope_lds(j, lane)];
    }
  }
}

template <int EPI, int WM, int WN, int KS = 2, int D = 1, bool Q4W = false>
hipError_t launch_mm_t(const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  if (a.nkb % KS) return hipErrorInvalidValue;
  dim3 grid((a.n_tiles + 4 * WN - 1) / (4 * WN), (a.M + 64 * WM - 1) / (64 * WM)), block(WM * WN * 64);
  if constexpr (WM * WN == 16) {
    if (a.kpart_n > 1) {
      // the reduction split over kpart_n workgroups per block, partials summed by a second launch
      dim3 sgrid(grid.x, grid.y, a.kpart_n), rgrid(grid.x, grid.y, WM * WN / 4);
      hipLaunchKernelGGL((mm_kernel<EPI, WM, WN, KS, D, true, Q4W>), sgrid, block, 0, st, a);
      if (tm)
        hipExtLaunchKernelGGL((mm_reduce_kernel<EPI, WM, WN>), rgrid, dim3(256), 0, st, tm->start,
                              tm->stop, 0, a);
      else
        hipLaunchKernelGGL((mm_reduce_kernel<EPI, WM, WN>), rgrid, dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.kpart_n > 1) return hipErrorInvalidValue;
  if (tm)
    hipExtLaunchKernelGGL((mm_kernel<EPI, WM, WN, KS, D, false, Q4W>), grid, block, 0, st, tm->start, tm->stop, 0, a);
  else
    hipLaunchKernelGGL((mm_kernel<EPI, WM, WN, KS, D, false, Q4W>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace gemm_detail

size_t launch_mm_partial_floats(int n_tiles, int M, int kpart_n) {
  // 256 x 256 blocks of 16 waves, each wave 16 fragments of 64 lanes x 4 floats
  return kpart_n > 1 ? (size_t)kpart_n * ((n_tiles + 15) / 16) * ((M + 255) / 256) * 16 * 16 * 64 * 4 : 0;
}

namespace gemm_detail {
template <bool Q4W>
hipError_t launch_mm_w(int epi, const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  if (a.kpart_n > 1) {
    // a projection too narrow for 256 x 256 blocks to fill the CUs: the same blocks with the
    // reduction split kpart_n ways (at least one stage each), partials summed by a second launch
    if (!a.kpart || a.kpart_n > a.nkb / 2) return hipErrorInvalidValue;
    switch (epi) {
      case EPI_STORE: return launch_mm_t<EPI_STORE, 4, 4, 2, 1, Q4W>(a, st, tm);
      case EPI_ROPE: return launch_mm_t<EPI_ROPE, 4, 4, 2, 1, Q4W>(a, st, tm);
      case EPI_SILU: return launch_mm_t<EPI_SILU, 4, 4, 2, 1, Q4W>(a, st, tm);
      case EPI_ARGMAX: return launch_mm_t<EPI_ARGMAX, 4, 4, 2, 1, Q4W>(a, st, tm);
      default: return hipErrorInvalidValue;
    }
  }
  if (epi == EPI_ARGMAX && a.n_tiles % 4) return hipErrorInvalidValue;  // whole 64-column units
  if (epi == EPI_SILU && a.n_tiles % 2) return hipErrorInvalidValue;    // gate/up pairs
  // 128 x 128 blocks; a projection too narrow to give every CU a block takes 64 x 128 blocks of
  // two waves instead (the model-width outputs: o and down)
  const int blocks = ((a.n_tiles + 7) / 8) * ((a.M + 127) / 128);
  const bool narrow = blocks < 256;
  switch (epi) {
    case EPI_STORE:
      return narrow ? launch_mm_t<EPI_STORE, 1, 2, 2, 1, Q4W>(a, st, tm)
                    : launch_mm_t<EPI_STORE, 2, 2, 2, 1, Q4W>(a, st, tm);
    case EPI_ROPE:
      return narrow ? launch_mm_t<EPI_ROPE, 1, 2, 2, 1, Q4W>(a, st, tm)
                    : launch_mm_t<EPI_ROPE, 2, 2, 2, 1, Q4W>(a, st, tm);
    // the wide projections (gate/up, LM head): 256 x 256 blocks of 16 waves, half the LDS and L2
    // bytes per product of 128 x 128 blocks (31B, 512 rows: prefill 303 -> 374 TFLOP/s; a
    // register ring of 2 to 4 stages in flight instead of one gained nothing)
    case EPI_SILU: return launch_mm_t<EPI_SILU, 4, 4, 2, 1, Q4W>(a, st, tm);
    case EPI_ARGMAX: return launch_mm_t<EPI_ARGMAX, 4, 4, 2, 1, Q4W>(a, st, tm);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace gemm_detail

hipError_t launch_mm(int epi, const GemmArgs& a, hipStream_t st, const LaunchTiming* tm) {
  using namespace gemm_detail;
  if (a.M <= 0 || a.n_tiles <= 0) return hipSuccess;
  if (a.nkb % 2 || (a.wq4 && a.nkb % 4)) return hipErrorInvalidValue;
  return a.wq4 ? launch_mm_w<true>(epi, a, st, tm) : launch_mm_w<false>(epi, a, st, tm);
}

}  // namespace specdec
