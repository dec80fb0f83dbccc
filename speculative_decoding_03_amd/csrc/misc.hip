// Small kernels of the step: embedding gather, fused argmax + acceptance + commit, KV commit,
// drafter input, cluster selection, draft finalisation, weight packing.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace specdec {

namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return s;
}

__device__ __forceinline__ void block_argmax(float& v, int& i, float* rv, int* ri) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  wave_argmax(v, i);
  __syncthreads();
  if (lane == 0) { rv[wid] = v; ri[wid] = i; }
  __syncthreads();
  v = rv[0];
  i = ri[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_combine(v, i, rv[w], ri[w]);
}

// x[m] = E[tokens[m]] (fp32 residual), xw[m] = x[m] * norm (the first layer's attention-norm
// weight, storage type; row-major or the quad layout) and the per-16-column sums of squares of
// x[m], from which the consumer forms the RMSNorm row scale.  Grid (d / 8 / 256 rounded up, M):
// each thread moves one run of 8 consecutive elements (contiguous in the packed table), and the
// two threads of a 16-column tile (adjacent lanes) add their sums with one lane exchange.
// One run of 8 consecutive weights of row n as fp32: dtype elements of a packed matrix, or the
// 4-bit block format (Q4).
template <typename T, bool Q4>
__device__ __forceinline__ void row_run8(const void* W, int n, int k8, int nkb, float (&v)[8]) {
  if constexpr (Q4) {
    q4_run8(reinterpret_cast<const uint8_t*>(W), n, k8, nkb, v);
  } else {
    Frag<T> f;
    load_frag<T>(f, reinterpret_cast<const T*>(W) + packed_offset(n, k8, nkb));
    frag_values<T>(f, v);
  }
}

template <typename T, bool Q4>
__global__ void __launch_bounds__(256) embed_kernel(const void* E, int nkb, int d, const int* tokens,
                                                    int M, float* x, float* ssq, T* xw, int xw_qx,
                                                    const float* norm, int vocab, int* err) {
  const int m = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;  // run of 8 elements in the row
  const int k8 = c * 8;
  int tok = tokens[m];
  if (tok < 0 || tok >= vocab) {
    if (c == 0) raise_error(err, ERRBIT_TOKEN);
    tok = 0;
  }
  float sq = 0.f;
  if (k8 < d) {
    float v[8], y[8];
    row_run8<T, Q4>(E, tok, k8, nkb, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = v[e] * norm[k8 + e];
      sq += v[e] * v[e];
    }
    f32x4* xo = reinterpret_cast<f32x4*>(x + (size_t)m * d + k8);
    xo[0] = f32x4{v[0], v[1], v[2], v[3]};
    xo[1] = f32x4{v[4], v[5], v[6], v[7]};
    Frag<T> o;
    to_frag<T>(o, y);
    u32x4* q = reinterpret_cast<u32x4*>(xw + x_offset(xw_qx, m, k8, d));
    if constexpr (sizeof(T) == 2) {
      q[0] = o.v;
    } else {
      q[0] = o.v[0];
      q[1] = o.v[1];
    }
  }
  const float tot = sq + dpp_f32<DPP_XOR1>(sq);  // runs 2t and 2t+1 form 16-column tile t
  if (k8 < d && (c & 1) == 0) ssq[(size_t)(k8 / TILE_N) * M + m] = tot;
}

// Per sequence: G[i] = argmax of row i over the LM-head partials; m = longest prefix with
// tokens[i+1] == G[i]; emit tokens[1..m] and G[m]; optionally commit (len += m+1, hid = X[m]).
__global__ void __launch_bounds__(1024) accept_kernel(
    const float* amax_val, const int* amax_idx, int n_parts, int ld_amax, int R,
    const int* tokens, int* out_tokens, int* n_emit, int* next_tok, int commit, int* len,
    float* hid, const float* X, int d, int* argmax_out, int* err) {
  // rows are reduced RG at a time: every thread's partial loads of the group are in flight
  // together, each wave reduces its share of every row, and after one barrier thread j combines
  // row j over the waves in wave order
  constexpr int RG = 8, NWV = 16;
  __shared__ float rv[RG][NWV];
  __shared__ int ri[RG][NWV];
  __shared__ int G[64];
  __shared__ int T[64];
  __shared__ int m_sh;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x >> 6;
  // the verify rows' tokens, requested with the first partials so that the acceptance scan
  // below reads them from LDS instead of one dependent memory round trip per accepted draft
  const int tok = tokens && (int)threadIdx.x < R ? tokens[b * R + threadIdx.x] : 0;
  for (int i0 = 0; i0 < R; i0 += RG) {
    float v[RG];
    int idx[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      v[j] = -INFINITY;
      idx[j] = 0x7fffffff;
    }
    if (n_parts % 4 == 0 && ld_amax % 4 == 0) {
      // four consecutive partials per 16-byte load (rows start 16-byte aligned); with n_parts
      // <= 4 * blockDim every row's loads are in flight together
      for (int p = 4 * threadIdx.x; p < n_parts; p += 4 * blockDim.x) {
        f32x4 pv[RG];
        int4 pi[RG];
#pragma unroll
        for (int j = 0; j < RG; ++j)
          if (i0 + j < R) {
            const size_t o = (size_t)(b * R + i0 + j) * ld_amax + p;
            pv[j] = *reinterpret_cast<const f32x4*>(amax_val + o);
            pi[j] = *reinterpret_cast<const int4*>(amax_idx + o);
          }
#pragma unroll
        for (int j = 0; j < RG; ++j)
          if (i0 + j < R) {
            argmax_combine(v[j], idx[j], pv[j][0], pi[j].x);
            argmax_combine(v[j], idx[j], pv[j][1], pi[j].y);
            argmax_combine(v[j], idx[j], pv[j][2], pi[j].z);
            argmax_combine(v[j], idx[j], pv[j][3], pi[j].w);
          }
      }
    } else {
      for (int p = threadIdx.x; p < n_parts; p += blockDim.x)
#pragma unroll
        for (int j = 0; j < RG; ++j)
          if (i0 + j < R) {
            const size_t o = (size_t)(b * R + i0 + j) * ld_amax + p;
            argmax_combine(v[j], idx[j], amax_val[o], amax_idx[o]);
          }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      if (i0 + j >= R) break;  // uniform
      wave_argmax(v[j], idx[j]);
      if (lane == 0) {
        rv[j][wid] = v[j];
        ri[j][wid] = idx[j];
      }
    }
    __syncthreads();
    const int j = threadIdx.x;
    if (j < RG && i0 + j < R) {
      float bv = rv[j][0];
      int bi = ri[j][0];
      for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_combine(bv, bi, rv[j][w], ri[j][w]);
      G[i0 + j] = bi;
      if (argmax_out) argmax_out[b * R + i0 + j] = bi;
    }
    __syncthreads();
  }
  if ((int)threadIdx.x < R) T[threadIdx.x] = tok;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int K = R - 1;
    int m = 0;
    if (tokens) {
      while (m < K && T[m + 1] == G[m]) ++m;
    }
    if (out_tokens) {
      for (int j = 0; j < m; ++j) out_tokens[b * R + j] = T[j + 1];
      out_tokens[b * R + m] = G[m];
      for (int j = m + 1; j < R; ++j) out_tokens[b * R + j] = -1;
    }
    if (n_emit) n_emit[b] = m + 1;
    if (next_tok) next_tok[b] = G[m];
    if (G[m] == 0x7fffffff) raise_error(err, ERRBIT_NAN);
    m_sh = m;
  }
  __syncthreads();
  if (commit) {
    const int m = m_sh;
    for (int k = threadIdx.x; k < d; k += blockDim.x)
      hid[(size_t)b * d + k] = X[((size_t)b * R + m) * d + k];
    if (threadIdx.x == 0) len[b] += m + 1;
  }
}

__global__ void __launch_bounds__(256) commit_kernel(const int* n_commit, int R, int* len,
                                                     float* hid, const float* X, int d, int* err) {
  const int b = blockIdx.x;
  const int n = n_commit[b];
  if (n < 1 || n > R) {
    if (threadIdx.x == 0) raise_error(err, ERRBIT_CAPACITY);
    return;
  }
  for (int k = threadIdx.x; k < d; k += blockDim.x)
    hid[(size_t)b * d + k] = X[((size_t)b * R + n - 1) * d + k];
  if (threadIdx.x == 0) len[b] += n;
}

// Per row of a prompt chunk: argmax over its LM-head partials (lowest index on ties), one
// workgroup per row.
__global__ void __launch_bounds__(256) rows_argmax_kernel(const float* amax_val, const int* amax_idx,
                                                          int n_parts, int ld, int* out) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x >> 6;
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (int p = threadIdx.x; p < n_parts; p += blockDim.x)
    argmax_combine(v, i, amax_val[(size_t)row * ld + p], amax_idx[(size_t)row * ld + p]);
  wave_argmax(v, i);
  if (lane == 0) {
    rv[wid] = v;
    ri[wid] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) argmax_combine(v, i, rv[w], ri[w]);
    out[row] = i;
  }
}

// Commit of a prompt chunk of n rows of one sequence: len += n, hid = the chunk's last hidden row.
__global__ void __launch_bounds__(256) commit_rows_kernel(int* len, float* hid, const float* xlast,
                                                          int d, int n) {
  for (int k = threadIdx.x; k < d; k += blockDim.x) hid[k] = xlast[k];
  if (threadIdx.x == 0) *len += n;
}

// u[b] = [ rms(h[b]) * norm_h ; rms(table[row(tok[b])]) * norm_e ] in the storage dtype.
// h is requested first, as 16-byte runs held in registers (when d <= 4 * HV * blockDim.x), so its
// latency overlaps the token -> table-row lookup; both sums of squares share one block reduction.
template <typename T, bool Q4>
__global__ void __launch_bounds__(256) draft_input_kernel(const float* h, const int* tok,
                                                          const void* table, int nkb_table,
                                                          const int* vocab_row, int vocab,
                                                          const float* norm_h, const float* norm_e,
                                                          int d, int Dd, float eps, T* u, int u_qx,
                                                          int h_div, int* err) {
  constexpr int HV = 8;
  __shared__ float red[2][16];
  __shared__ float ebuf[1024];
  const int b = blockIdx.x, t = threadIdx.x;
  const int lane = t & (WAVE - 1), wid = t >> 6;
  const float* hb = h + (size_t)(b / h_div) * d;  // h_div rows share one hidden input
  const bool hreg = d % 4 == 0 && d <= 4 * HV * (int)blockDim.x;
  f32x4 hv[HV];
  if (hreg) {
#pragma unroll
    for (int i = 0; i < HV; ++i) {
      const int k = (t + i * (int)blockDim.x) * 4;
      hv[i] = k < d ? *reinterpret_cast<const f32x4*>(hb + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  int c = tok[b];
  if (c < 0 || c >= vocab) {
    if (t == 0) raise_error(err, ERRBIT_TOKEN);
    c = 0;
  }
  const int row = vocab_row[c];
  float sse = 0.f;
  for (int k8 = t * 8; k8 < Dd; k8 += blockDim.x * 8) {
    float v[8];
    row_run8<T, Q4>(table, row, k8, nkb_table, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ebuf[k8 + e] = v[e];
      sse += v[e] * v[e];
    }
  }
  float ssh = 0.f;
  if (hreg) {
#pragma unroll
    for (int i = 0; i < HV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) ssh += hv[i][e] * hv[i][e];
  } else {
    for (int k = t; k < d; k += blockDim.x) ssh += hb[k] * hb[k];
  }
  ssh = wave_sum(ssh);
  sse = wave_sum(sse);
  if (lane == 0) {
    red[0][wid] = ssh;
    red[1][wid] = sse;
  }
  __syncthreads();
  ssh = 0.f;
  sse = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    ssh += red[0][w];
    sse += red[1][w];
  }
  const float rh = 1.0f / sqrtf(ssh / (float)d + eps);
  const float re = 1.0f / sqrtf(sse / (float)Dd + eps);
  if (hreg) {
#pragma unroll
    for (int i = 0; i < HV; ++i) {
      const int k = (t + i * (int)blockDim.x) * 4;
      if (k < d)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Elem<T>::store(u + x_offset(u_qx, b, k + e, d + Dd), hv[i][e] * rh * norm_h[k + e]);
    }
  } else {
    for (int k = t; k < d; k += blockDim.x)
      Elem<T>::store(u + x_offset(u_qx, b, k, d + Dd), hb[k] * rh * norm_h[k]);
  }
  for (int k = t; k < Dd; k += blockDim.x)
    Elem<T>::store(u + x_offset(u_qx, b, d + k, d + Dd), ebuf[k] * re * norm_e[k]);
}

// Selects the k_c best clusters of z[b] (ties -> lower cluster id) and lists their tiles as
// argmax units: selected cluster r of sequence b owns units (b*k_c + r)*upc .. +upc-1.
__global__ void __launch_bounds__(256) cluster_select_kernel(const float* z, int Nc, int k_c,
                                                             int tiles_per_cluster, int upc,
                                                             int* unit_tile, int* unit_row,
                                                             int* err) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int b = blockIdx.x;
  const float* zb = z + (size_t)b * Nc;
  const int tiles_per_unit = tiles_per_cluster / upc;
  if (k_c == 1) {
    float v = -INFINITY;
    int idx = 0x7fffffff;
    for (int c = threadIdx.x; c < Nc; c += blockDim.x) argmax_combine(v, idx, zb[c], c);
    block_argmax(v, idx, rv, ri);
    if (idx < 0 || idx >= Nc) {  // only when every score is NaN
      if (threadIdx.x == 0) raise_error(err, ERRBIT_NAN);
      idx = 0;
    }
    if (threadIdx.x < upc) {
      const int u = b * upc + threadIdx.x;
      unit_tile[u] = idx * tiles_per_cluster + threadIdx.x * tiles_per_unit;
      unit_row[u] = b;
    }
    return;
  }
  for (int c = threadIdx.x; c < Nc; c += blockDim.x) {
    const float zc = zb[c];
    int rank = 0;
    for (int c2 = 0; c2 < Nc; ++c2) {
      const float z2 = zb[c2];
      rank += (z2 > zc) || (z2 == zc && c2 < c);
    }
    if (rank < k_c) {
      for (int q = 0; q < upc; ++q) {
        const int u = (b * k_c + rank) * upc + q;
        unit_tile[u] = c * tiles_per_cluster + q * tiles_per_unit;
        unit_row[u] = b;
      }
    }
  }
}

// Mixture-of-experts routing (one workgroup): per row, the top_k router logits by repeated
// wave argmax (ties -> lower expert id) and their softmax weights; then, per expert, the rows
// routed to it in ascending row order, and the ascending list of experts that received a row.
// The per-expert lists come from a bit set of rows per expert: a (row, expert) pair's place in
// its expert's list is the number of lower rows routed to that expert, so every pair writes its
// own entry with no ordering between threads.
constexpr int MOE_MAX_M = 64, MOE_MAX_E = 256, MOE_MAX_K = 16;

constexpr int MOE_ROUTE_WAVES = 16;

__global__ void __launch_bounds__(MOE_ROUTE_WAVES * 64) moe_route_kernel(const float* logits, int M, int E,
                                                        int top_k, int* xrow, int* orow,
                                                        float* wt, int* group_list,
                                                        int* n_groups, int* usage, int* err) {
  __shared__ int sel[MOE_MAX_M][MOE_MAX_K];
  __shared__ float selw[MOE_MAX_M][MOE_MAX_K];
  __shared__ unsigned long long rows_of[MOE_MAX_E];  // bit m: row m is routed to the expert
  __shared__ int wtot[MOE_ROUTE_WAVES];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) rows_of[e] = 0ull;
  // Every logit of the wave's rows is requested before any is used (one memory round trip); a
  // row or expert past the call reads a valid entry, masked below.
  constexpr int RPW = MOE_MAX_M / MOE_ROUTE_WAVES;  // rows per wave
  constexpr int EPL = MOE_MAX_E / WAVE;             // logits per lane and row
  __shared__ float wsel[MOE_ROUTE_WAVES][MOE_MAX_K];
  float lv[RPW][EPL];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      lv[i][j] = logits[(size_t)min(wid + MOE_ROUTE_WAVES * i, M - 1) * E + min(lane + WAVE * j, E - 1)];
  const unsigned long long below = (1ull << lane) - 1ull;  // lanes under this one
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int m = wid + MOE_ROUTE_WAVES * i;
    if (m >= M) break;  // wave-uniform
    // Selection of the top_k logits, larger first and the lower expert id on equal values, as
    // one threshold: the top_k-th largest key of the order-preserving integer keys (NaN as -inf,
    // -0 as +0), found bit by bit from the wave's counts; then the experts with equal keys are
    // taken in ascending id up to top_k.  Expert e = lane + 64 j sits in slot j of its lane.
    uint32_t key[EPL];
    float v[EPL];
    bool ok[EPL], nan = false;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const float x = lv[i][j];
      ok[j] = lane + WAVE * j < E;
      nan |= ok[j] && (x != x);
      v[j] = x == x ? x + 0.0f : -INFINITY;  // + 0 turns -0 into +0
      const uint32_t u = __float_as_uint(v[j]);
      key[j] = ok[j] ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
    }
    if (nan) raise_error(err, ERRBIT_NAN);
    auto count_ge = [&](uint32_t t) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) c += __popcll(__ballot(ok[j] && key[j] >= t));
      return c;
    };
    uint32_t T = 0u;  // the largest threshold with at least top_k keys at or above it
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      if (count_ge(cand) >= top_k) T = cand;
    }
    int above = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) above += __popcll(__ballot(ok[j] && key[j] > T));
    const int need = top_k - above;  // experts with key == T taken, lowest ids first
    bool pick[EPL];
    int tie_before = 0;  // equal keys at lower expert ids
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const bool tie = ok[j] && key[j] == T;
      const unsigned long long b = __ballot(tie);
      pick[j] = (ok[j] && key[j] > T) || (tie && tie_before + __popcll(b & below) < need);
      tie_before += __popcll(b);
    }
    // the selected experts in ascending id (slot 0 lanes first): their rank is their place
    float vmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) vmax = fmaxf(vmax, pick[j] ? v[j] : -INFINITY);
    vmax = wave_max(vmax);  // the largest selected logit
    int before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const unsigned long long b = __ballot(pick[j]);
      if (pick[j]) {
        const int rank = before + __popcll(b & below);
        const float w = expf(v[j] - vmax);
        sel[m][rank] = lane + WAVE * j;
        wsel[wid][rank] = w;
      }
      before += __popcll(b);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the weights' sum in rank order, then each weight divided by it
    float sum = 0.f;
    for (int k = 0; k < top_k; ++k) sum += wsel[wid][k];
    if (lane < top_k) selw[m][lane] = wsel[wid][lane] / sum;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();
  const int P = M * top_k;  // (row, rank) pairs, at most MOE_MAX_M * MOE_MAX_K = 1024
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int m = p / top_k;
    atomicOr(&rows_of[sel[m][p - m * top_k]], 1ull << m);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int m = p / top_k, k = p - m * top_k;
    const int e = sel[m][k];
    const int c = __popcll(rows_of[e] & ((1ull << m) - 1ull));  // lower rows of this expert
    xrow[(size_t)e * M + c] = m;
    orow[(size_t)e * M + c] = p;
    wt[(size_t)e * M + c] = selw[m][k];
  }
  for (int q = threadIdx.x; q < E * M; q += blockDim.x) {
    const int e = q / M;
    if (q - e * M >= __popcll(rows_of[e])) {  // past the expert's rows
      xrow[q] = -1;
      orow[q] = -1;
      wt[q] = 0.f;
    }
  }
  const int e = threadIdx.x;
  const bool used = e < E && rows_of[e] != 0ull;
  const unsigned long long mask = __ballot(used);
  if (lane == 0) wtot[wid] = __popcll(mask);
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wid; ++w) off += wtot[w];
  if (used) group_list[off + __popcll(mask & ((1ull << lane) - 1ull))] = e;
  if (threadIdx.x == 0) {
    int ng = 0;
    for (int w = 0; w < MOE_ROUTE_WAVES; ++w) ng += wtot[w];
    n_groups[0] = ng;
    if (usage) usage[0] += ng;  // one writer: the launches of a layer are ordered on the stream
  }
}

// Reduces a sequence's head partials to the drafted token, records it as the next sub-step's
// input, and applies the optional injected replacement for slot j at position len[b] + j.
__global__ void __launch_bounds__(256) draft_finalize_kernel(
    const float* amax_val, const int* amax_idx, int ld_amax, int parts_per_seq, int seq_offset,
    int K, int j, const int* len, const int* inject, int inj_stride, int* drafts, int* dtok,
    const int* cur_tok, int* vtok, int* err) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int b = blockIdx.x;
  const int u0 = b * seq_offset;
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int p = threadIdx.x; p < parts_per_seq; p += blockDim.x)
    argmax_combine(v, idx, amax_val[(size_t)b * ld_amax + u0 + p], amax_idx[(size_t)b * ld_amax + u0 + p]);
  block_argmax(v, idx, rv, ri);
  if (threadIdx.x == 0) {
    if (idx == 0x7fffffff) {
      raise_error(err, ERRBIT_NAN);
      idx = 0;
    }
    dtok[b] = idx;
    int out = idx;
    if (inject) {
      const long long slot = (long long)(len[b] + j) * K + (j - 1);
      if (slot >= 0 && slot < inj_stride) {
        const int r = inject[(size_t)b * inj_stride + slot];
        if (r >= 0) out = r;
      }
    }
    drafts[b * K + (j - 1)] = out;
    if (vtok) {  // the verify input row [c0, d1..dK]
      if (j == 1) vtok[b * (K + 1)] = cur_tok[b];
      vtok[b * (K + 1) + j] = out;
    }
  }
}

// dst (packed tiles) <- src (logical row-major [N][Kd]).
//   kind 0: plain; kind 1: rotary heads of hd with pairs (i, i+hd/2) made adjacent;
//   kind 2: gate rows [0, F) and up rows [F, 2F) interleaved tile by tile (F = split_rows), in
//   each group of 2F rows (N a multiple of 2F: stacked expert matrices).
template <typename T>
__global__ void pack_kernel(const T* src, T* dst, int N, int Kd, int kind, int hd, int F) {
  const size_t total = (size_t)N * Kd;
  const int nkb = Kd / TILE_K;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(e / Kd);
    const int k = (int)(e - (size_t)n * Kd);
    int sr = n;
    if (kind == 1) {
      const int head = n / hd, p = n - head * hd;
      sr = head * hd + (p >> 1) + (p & 1) * (hd >> 1);
    } else if (kind == 2) {
      const int g = n / (2 * F), nl = n - g * 2 * F;
      const int tile = nl >> 4;
      sr = g * 2 * F + (tile & 1) * F + (tile >> 1) * TILE_N + (nl & 15);
    }
    dst[packed_offset(n, k, nkb)] = src[(size_t)sr * Kd + k];
  }
}

// 4-bit block matrix from codes [N][Kd] (bytes, low 4 bits used) and fp16 steps [N][Kd/32], rows
// permuted as pack_kernel does.  One thread per (row, run of 8 codes): it writes the run's code
// dword, and the first run of each 32-block also writes the block's step.
__global__ void pack_q4_kernel(const uint8_t* q, const uint16_t* steps, uint8_t* dst, int N, int Kd,
                               int kind, int hd, int F) {
  const int runs = Kd / 8;
  const size_t total = (size_t)N * runs;
  const int nkb = Kd / TILE_K;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(e / runs);
    const int k0 = (int)(e - (size_t)n * runs) * 8;
    int sr = n;
    if (kind == 1) {
      const int head = n / hd, p = n - head * hd;
      sr = head * hd + (p >> 1) + (p & 1) * (hd >> 1);
    } else if (kind == 2) {
      const int g = n / (2 * F), nl = n - g * 2 * F;
      const int tile = nl >> 4;
      sr = g * 2 * F + (tile & 1) * F + (tile >> 1) * TILE_N + (nl & 15);
    }
    const uint8_t* src = q + (size_t)sr * Kd + k0;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) c |= (uint32_t)(src[i] & 15u) << ((i & 1) * 16 + (i >> 1) * 4);
    uint8_t* blk = dst + q4_block_offset(n, k0, nkb);
    const int kb = (k0 >> 5) & 3, kg = (k0 >> 3) & 3, r = n & 15;
    *reinterpret_cast<uint32_t*>(blk + (kg * 16 + r) * 16 + kb * 4) = c;
    if (kg == 0)
      *reinterpret_cast<uint16_t*>(blk + Q4_CODE_BYTES + r * 8 + kb * 2) =
          steps[(size_t)sr * (Kd / 32) + (k0 >> 5)];
  }
}

// ---- tree drafts ----

// Inject-or-keep of one drafted tree node: the table entry (len + depth) * n_slots + slot, when
// it lies in the table and is not -1, replaces the token shown to the verify.
__device__ __forceinline__ int inject_node(const int* inject, int inj_stride, int b, int len,
                                           int depth, int n_slots, int slot, int tok) {
  if (!inject) return tok;
  const long long e = (long long)(len + depth) * n_slots + slot;
  if (e < 0 || e >= inj_stride) return tok;
  const int r = inject[(size_t)b * inj_stride + e];
  return r >= 0 ? r : tok;
}

// The first level of a tree draft: the w best tokens of sequence b among the rows the head scored
// (scores[b][row], by table row): for the clustered head the units_per_seq listed units of
// sequence b (unit_tile[b*units_per_seq + i] = first tile, rows_per_unit rows each), for the full
// head (unit_tile null) every row.  Ranked by score, then lower vocabulary id.  Writes the tree's
// root (the current token) and nodes 1..w (after injection), and the branches' raw tokens (the
// next sub-step's inputs).
__global__ void __launch_bounds__(1024) tree_top_kernel(
    const float* scores, int vocab, const int* unit_tile, int units_per_seq, int rows_per_unit,
    const int* row_vocab, int w, int D, const int* cur_tok, const int* len, const int* inject,
    int inj_stride, int* tree_tok, int* raw, int* err) {
  __shared__ float rv[16];
  __shared__ int ri[16];
  __shared__ int chosen[16];
  const int b = blockIdx.x;
  const int n_rows = unit_tile ? units_per_seq * rows_per_unit : vocab;
  const float* sc = scores + (size_t)b * vocab;
  const int n_nodes = 1 + w * D;
  for (int k = 0; k < w; ++k) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int i = threadIdx.x; i < n_rows; i += blockDim.x) {
      const int row = unit_tile ? unit_tile[(size_t)b * units_per_seq + i / rows_per_unit] * TILE_N +
                                      i % rows_per_unit
                                : i;
      const int vid = row_vocab[row];
      bool taken = false;
      for (int q = 0; q < k; ++q) taken |= chosen[q] == vid;
      if (!taken) argmax_combine(v, id, sc[row], vid);
    }
    block_argmax(v, id, rv, ri);
    if (threadIdx.x == 0) {
      if (id == 0x7fffffff) {  // fewer candidates than branches, or every score NaN
        raise_error(err, ERRBIT_NAN);
        id = 0;
      }
      chosen[k] = id;
    }
    __syncthreads();
  }
  if (threadIdx.x < w) {
    const int k = threadIdx.x;
    raw[b * w + k] = chosen[k];
    tree_tok[(size_t)b * n_nodes + 1 + k] =
        inject_node(inject, inj_stride, b, len[b], 1, w * D, k, chosen[k]);
  }
  if (threadIdx.x == 0) tree_tok[(size_t)b * n_nodes] = cur_tok[b];
}

// Levels 2..D of a tree draft: row r = (sequence b, branch k) reduces its head partials to its
// token, which feeds the branch's next sub-step, and writes node 1 + w*(depth-1) + k.
__global__ void __launch_bounds__(256) tree_finalize_kernel(
    const float* amax_val, const int* amax_idx, int ld_amax, int parts, int seq_offset, int w,
    int D, int depth, const int* len, const int* inject, int inj_stride, int* tree_tok, int* raw,
    int* err) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int r = blockIdx.x;
  const int b = r / w, k = r - b * w;
  const int u0 = r * seq_offset;
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int p = threadIdx.x; p < parts; p += blockDim.x)
    argmax_combine(v, idx, amax_val[(size_t)r * ld_amax + u0 + p], amax_idx[(size_t)r * ld_amax + u0 + p]);
  block_argmax(v, idx, rv, ri);
  if (threadIdx.x == 0) {
    if (idx == 0x7fffffff) {
      raise_error(err, ERRBIT_NAN);
      idx = 0;
    }
    raw[r] = idx;
    const int node = 1 + w * (depth - 1) + k;
    tree_tok[(size_t)b * (1 + w * D) + node] =
        inject_node(inject, inj_stride, b, len[b], depth, w * D, node - 1, idx);
  }
}

// Acceptance over a token tree (nodes in topological order, parent[0] = -1): G[i] = argmax of
// node i's row; the longest root path on which every node's token is G at its parent (among
// equally long ones the lower node index at the first difference) is accepted; emit its tokens
// and the target's token at its end.  With
// commit: len += m + 1, hid = hidden of the path's last node, and the path's nodes are recorded
// (path[b][0] = old length, path[b][1..m] = node indices) for the cache compaction.
struct TreeShape {
  int n;
  int8_t parent[64];
};
constexpr int TREE_MAX_DEPTH = 16;  // longest accepted path the compaction moves

__global__ void __launch_bounds__(1024) tree_accept_kernel(
    const float* amax_val, const int* amax_idx, int n_parts, int ld_amax, TreeShape tr,
    const int* tokens, int* out_tokens, int out_ld, int* n_emit, int* next_tok, int commit,
    int* len, float* hid, const float* X, int d, int* path, int* err) {
  constexpr int NWV = 16;
  __shared__ float rv[NWV];
  __shared__ int ri[NWV];
  __shared__ int G[64];
  __shared__ int endn, mm;
  const int b = blockIdx.x, R = tr.n;
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x >> 6;
  for (int i = 0; i < R; ++i) {
    float v = -INFINITY;
    int idx = 0x7fffffff;
    for (int p = threadIdx.x; p < n_parts; p += blockDim.x) {
      const size_t o = (size_t)(b * R + i) * ld_amax + p;
      argmax_combine(v, idx, amax_val[o], amax_idx[o]);
    }
    wave_argmax(v, idx);
    if (lane == 0) {
      rv[wid] = v;
      ri[wid] = idx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = rv[0];
      int bi = ri[0];
      for (int w2 = 1; w2 < (int)(blockDim.x >> 6); ++w2) argmax_combine(bv, bi, rv[w2], ri[w2]);
      G[i] = bi;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    // longest agreeing path below each node, children visited in ascending index so that the
    // lowest-index child wins among equally long continuations (nodes are in topological order)
    int8_t best_len[64], best_child[64];
    for (int i = R - 1; i >= 0; --i) {
      best_len[i] = 0;
      best_child[i] = -1;
      for (int c = i + 1; c < R; ++c)
        if (tr.parent[c] == i && tokens[b * R + c] == G[i] && best_len[c] + 1 > best_len[i]) {
          best_len[i] = (int8_t)(best_len[c] + 1);
          best_child[i] = (int8_t)c;
        }
    }
    int cur = 0, m = 0;
    int nodes[64];
    while (best_child[cur] >= 0) {
      const int nxt = best_child[cur];
      out_tokens[b * out_ld + m] = tokens[b * R + nxt];
      nodes[m] = nxt;
      ++m;
      cur = nxt;
    }
    out_tokens[b * out_ld + m] = G[cur];
    for (int j = m + 1; j < out_ld; ++j) out_tokens[b * out_ld + j] = -1;
    if (n_emit) n_emit[b] = m + 1;
    if (next_tok) next_tok[b] = G[cur];
    if (G[cur] == 0x7fffffff) raise_error(err, ERRBIT_NAN);
    if (commit) {
      path[b * 65] = len[b];
      path[b * 65 + 1] = m;
      for (int j = 0; j < m; ++j) path[b * 65 + 2 + j] = nodes[j];
    }
    endn = cur;
    mm = m;
  }
  __syncthreads();
  if (commit) {
    const int e = endn;
    for (int k = threadIdx.x; k < d; k += blockDim.x)
      hid[(size_t)b * d + k] = X[((size_t)b * R + e) * d + k];
    if (threadIdx.x == 0) len[b] += mm + 1;
  }
}

// Moves the cache entries of an accepted tree path to consecutive slots: for path node j (1..m,
// at depth j) slot old_len + node_j -> old_len + j, in every layer, KV head and element.  Each
// thread reads every move of its element before it writes any, so a slot that is both a source
// and a destination is read first.  K is [pos][hd], V transposed [hd][pos].
template <typename T>
__global__ void __launch_bounds__(256) kv_compact_kernel(T* kc, T* vc, const int* path, int L,
                                                         int Bmax, int hkv, int hd, int max_ctx) {
  const int b = blockIdx.y;
  const int m = path[b * 65 + 1];
  if (m <= 0 || m > TREE_MAX_DEPTH) return;
  const int len0 = path[b * 65];
  // every source slot (and so every destination, which is lower) must lie in the cache; a length
  // beyond it was already flagged by the verify's kernels, and nothing is moved
  for (int j = 0; j < m; ++j) {
    const int node = path[b * 65 + 2 + j];
    if (len0 < 0 || node < j + 1 || len0 + node >= max_ctx) return;
  }
  const size_t per = (size_t)L * hkv * hd;  // elements of one sequence's moves per slot
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < per;
       e += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % hd);
    const size_t lg = e / hd;  // layer * hkv + g
    const int g = (int)(lg % hkv), l = (int)(lg / hkv);
    const size_t head = (((size_t)l * Bmax + b) * hkv + g);
    T* kh = kc + head * max_ctx * hd;
    T* vh = vc + head * hd * max_ctx + (size_t)c * max_ctx;
    T kv[TREE_MAX_DEPTH], vv[TREE_MAX_DEPTH];
#pragma unroll
    for (int j = 0; j < TREE_MAX_DEPTH; ++j)
      if (j < m) {
        const int src = len0 + path[b * 65 + 2 + j];
        kv[j] = kh[(size_t)src * hd + c];
        vv[j] = vh[src];
      }
#pragma unroll
    for (int j = 0; j < TREE_MAX_DEPTH; ++j)
      if (j < m) {
        const int dst = len0 + 1 + j;
        kh[(size_t)dst * hd + c] = kv[j];
        vh[dst] = vv[j];
      }
  }
}

__global__ void __launch_bounds__(256) trace_state_kernel(const float* x, const float* ssq, int B,
                                                          int n, const float* norm, float eps,
                                                          float* out, int ld_out) {
  __shared__ float rs;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int t = 0; t < n / TILE_N; ++t) s += ssq[(size_t)t * B + b];
    rs = 1.0f / sqrtf(s / (float)n + eps);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < n; k += blockDim.x)
    out[(size_t)b * ld_out + k] = x[(size_t)b * n + k] * rs * norm[k];
}

__global__ void copy_rows_kernel(uint32_t* dst, int ld_dst, const uint32_t* src, int ld_src,
                                 int cols) {
  const int r = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < cols; c += gridDim.x * blockDim.x)
    dst[(size_t)r * ld_dst + c] = src[(size_t)r * ld_src + c];
}

__global__ void fill_i32_kernel(int* p, int v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_embed(int dtype, const void* E, int nkb, int d, const int* tokens, int M,
                        float* x, float* ssq, void* xw, int xw_qx, const float* norm, int vocab,
                        int* err, hipStream_t st, int e_q4) {
  if (M <= 0) return hipSuccess;
  if (xw_qx && M > 4) return hipErrorInvalidValue;
  if (d % TILE_N) return hipErrorInvalidValue;
  if (e_q4 && (dtype != DT_BF16 || nkb % 4)) return hipErrorInvalidValue;
  const dim3 grid((d / 8 + 255) / 256, M);
  if (e_q4)
    hipLaunchKernelGGL((embed_kernel<bf16_t, true>), grid, dim3(256), 0, st, E, nkb, d, tokens, M,
                       x, ssq, (bf16_t*)xw, xw_qx, norm, vocab, err);
  else if (dtype == DT_BF16)
    hipLaunchKernelGGL((embed_kernel<bf16_t, false>), grid, dim3(256), 0, st, E, nkb, d, tokens, M,
                       x, ssq, (bf16_t*)xw, xw_qx, norm, vocab, err);
  else
    hipLaunchKernelGGL((embed_kernel<float, false>), grid, dim3(256), 0, st, E, nkb, d, tokens, M,
                       x, ssq, (float*)xw, xw_qx, norm, vocab, err);
  return hipGetLastError();
}

hipError_t launch_accept(const float* amax_val, const int* amax_idx, int n_parts, int ld_amax,
                         int B, int R, const int* tokens, int* out_tokens, int* n_emit,
                         int* next_tok, int commit, int* len, float* hid, const float* X, int d,
                         int* argmax_out, int* err, hipStream_t st) {
  if (R < 1 || R > 64) return hipErrorInvalidValue;  // the kernel's row arrays hold 64
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(1024), 0, st, amax_val, amax_idx, n_parts,
                     ld_amax, R, tokens, out_tokens, n_emit, next_tok, commit, len, hid, X, d,
                     argmax_out, err);
  return hipGetLastError();
}

hipError_t launch_commit(const int* n_commit, int B, int R, int* len, float* hid, const float* X,
                         int d, int* err, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(256), 0, st, n_commit, R, len, hid, X, d, err);
  return hipGetLastError();
}

hipError_t launch_rows_argmax(const float* amax_val, const int* amax_idx, int n_parts, int ld,
                              int rows, int* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rows_argmax_kernel, dim3(rows), dim3(256), 0, st, amax_val, amax_idx, n_parts,
                     ld, out);
  return hipGetLastError();
}

hipError_t launch_commit_rows(int* len, float* hid, const float* xlast, int d, int n,
                              hipStream_t st) {
  hipLaunchKernelGGL(commit_rows_kernel, dim3(1), dim3(256), 0, st, len, hid, xlast, d, n);
  return hipGetLastError();
}

hipError_t launch_draft_input(int dtype, const float* h, const int* tok, const void* table,
                              int nkb_table, const int* vocab_row, int vocab, const float* norm_h,
                              const float* norm_e, int d, int Dd, float eps, void* u, int u_qx,
                              int B, int* err, hipStream_t st, int h_div, int t_q4) {
  if (u_qx && B > 4) return hipErrorInvalidValue;
  if (h_div < 1) return hipErrorInvalidValue;
  if (t_q4 && (dtype != DT_BF16 || nkb_table % 4)) return hipErrorInvalidValue;
  if (t_q4)
    hipLaunchKernelGGL((draft_input_kernel<bf16_t, true>), dim3(B), dim3(256), 0, st, h, tok, table,
                       nkb_table, vocab_row, vocab, norm_h, norm_e, d, Dd, eps, (bf16_t*)u, u_qx,
                       h_div, err);
  else if (dtype == DT_BF16)
    hipLaunchKernelGGL((draft_input_kernel<bf16_t, false>), dim3(B), dim3(256), 0, st, h, tok,
                       table, nkb_table, vocab_row, vocab, norm_h, norm_e, d, Dd, eps, (bf16_t*)u,
                       u_qx, h_div, err);
  else
    hipLaunchKernelGGL((draft_input_kernel<float, false>), dim3(B), dim3(256), 0, st, h, tok,
                       table, nkb_table, vocab_row, vocab, norm_h, norm_e, d, Dd, eps, (float*)u,
                       u_qx, h_div, err);
  return hipGetLastError();
}

hipError_t launch_cluster_select(const float* z, int Nc, int k_c, int B, int tiles_per_cluster,
                                 int units_per_cluster, int* unit_tile, int* unit_row, int* err,
                                 hipStream_t st) {
  hipLaunchKernelGGL(cluster_select_kernel, dim3(B), dim3(256), 0, st, z, Nc, k_c,
                     tiles_per_cluster, units_per_cluster, unit_tile, unit_row, err);
  return hipGetLastError();
}

hipError_t launch_moe_route(const float* logits, int M, int E, int top_k, int* xrow, int* orow,
                            float* wt, int* group_list, int* n_groups, int* usage, int* err,
                            hipStream_t st) {
  if (M < 1 || M > MOE_MAX_M || E < 1 || E > MOE_MAX_E || top_k < 1 || top_k > MOE_MAX_K ||
      top_k > E)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(MOE_ROUTE_WAVES * 64), 0, st, logits, M, E, top_k, xrow, orow,
                     wt, group_list, n_groups, usage, err);
  return hipGetLastError();
}

hipError_t launch_draft_finalize(const float* amax_val, const int* amax_idx, int ld_amax,
                                 int parts_per_seq, int seq_offset, int B, int K, int j,
                                 const int* len, const int* inject, int inj_stride, int* drafts,
                                 int* dtok, const int* cur_tok, int* vtok, int* err,
                                 hipStream_t st) {
  hipLaunchKernelGGL(draft_finalize_kernel, dim3(B), dim3(256), 0, st, amax_val, amax_idx,
                     ld_amax, parts_per_seq, seq_offset, K, j, len, inject, inj_stride, drafts,
                     dtok, cur_tok, vtok, err);
  return hipGetLastError();
}

hipError_t launch_pack(int dtype, const void* src, void* dst, int N, int Kd, int kind, int hd,
                       int split_rows, hipStream_t st) {
  const size_t total = (size_t)N * Kd;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(pack_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)src,
                       (bf16_t*)dst, N, Kd, kind, hd, split_rows);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)src,
                       (float*)dst, N, Kd, kind, hd, split_rows);
  return hipGetLastError();
}

hipError_t launch_pack_q4(const uint8_t* q, const uint16_t* steps, void* dst, int N, int Kd,
                          int kind, int hd, int split_rows, hipStream_t st) {
  const size_t total = (size_t)N * (Kd / 8);
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  hipLaunchKernelGGL(pack_q4_kernel, dim3(blocks), dim3(256), 0, st, q, steps, (uint8_t*)dst, N, Kd,
                     kind, hd, split_rows);
  return hipGetLastError();
}

// Rotary (cos, sin) of every position and pair: angle pos * theta^(-2i/hd) for i < hd/2, formed and
// reduced to [-pi, pi] in fp64, then sine and cosine in fp32.  One table per context; the q/k
// projection epilogues read it instead of evaluating the angle per element.
__global__ void rope_table_kernel(float2* t, int hd, int max_ctx, float theta) {
  const int half = hd / 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)max_ctx * half) return;
  const int pos = (int)(idx / half), i = (int)(idx - (size_t)pos * half);
  const double inv_freq = pow((double)theta, -2.0 * (double)i / (double)hd);
  const double ang = (double)pos * inv_freq;
  const double turns = rint(ang * (0.5 / M_PI));
  const float r = (float)fma(-turns, 2.0 * M_PI, ang);
  float sn, cs;
  sincosf(r, &sn, &cs);
  t[idx] = make_float2(cs, sn);
}

hipError_t launch_rope_table(float2* t, int hd, int max_ctx, float theta, hipStream_t st) {
  const size_t n = (size_t)max_ctx * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, t, hd,
                     max_ctx, theta);
  return hipGetLastError();
}

hipError_t launch_tree_top(const float* scores, int vocab, const int* unit_tile, int units_per_seq,
                           int rows_per_unit, const int* row_vocab, int B, int w, int D,
                           const int* cur_tok, const int* len, const int* inject, int inj_stride,
                           int* tree_tok, int* raw, int* err, hipStream_t st) {
  if (w < 1 || w > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_top_kernel, dim3(B), dim3(1024), 0, st, scores, vocab, unit_tile,
                     units_per_seq, rows_per_unit, row_vocab, w, D, cur_tok, len, inject,
                     inj_stride, tree_tok, raw, err);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(const float* amax_val, const int* amax_idx, int ld_amax, int parts,
                                int seq_offset, int rows, int w, int D, int depth, const int* len,
                                const int* inject, int inj_stride, int* tree_tok, int* raw,
                                int* err, hipStream_t st) {
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(rows), dim3(256), 0, st, amax_val, amax_idx,
                     ld_amax, parts, seq_offset, w, D, depth, len, inject, inj_stride, tree_tok,
                     raw, err);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const float* amax_val, const int* amax_idx, int n_parts, int ld_amax,
                              int B, int n_nodes, const int8_t* parent, const int* tokens,
                              int* out_tokens, int out_ld, int* n_emit, int* next_tok, int commit,
                              int* len, float* hid, const float* X, int d, int* path, int* err,
                              hipStream_t st) {
  if (n_nodes < 1 || n_nodes > 64) return hipErrorInvalidValue;
  TreeShape tr{};
  tr.n = n_nodes;
  for (int i = 0; i < n_nodes; ++i) tr.parent[i] = parent[i];
  hipLaunchKernelGGL(tree_accept_kernel, dim3(B), dim3(1024), 0, st, amax_val, amax_idx, n_parts,
                     ld_amax, tr, tokens, out_tokens, out_ld, n_emit, next_tok, commit, len, hid,
                     X, d, path, err);
  return hipGetLastError();
}

struct TreeDesc {
  int n;
  uint8_t depth[64];
  uint64_t mask[64];
};

__global__ void tree_desc_kernel(TreeDesc t, uint64_t* mask_out, uint8_t* depth_out) {
  const int i = threadIdx.x;
  if (i < t.n) {
    mask_out[i] = t.mask[i];
    depth_out[i] = t.depth[i];
  }
}

hipError_t launch_tree_desc(int n, const uint64_t* mask, const uint8_t* depth, uint64_t* mask_out,
                            uint8_t* depth_out, hipStream_t st) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  TreeDesc t{};
  t.n = n;
  for (int i = 0; i < n; ++i) {
    t.mask[i] = mask[i];
    t.depth[i] = depth[i];
  }
  hipLaunchKernelGGL(tree_desc_kernel, dim3(1), dim3(64), 0, st, t, mask_out, depth_out);
  return hipGetLastError();
}

hipError_t launch_kv_compact(int dtype, void* kc, void* vc, const int* path, int L, int B,
                             int Bmax, int hkv, int hd, int max_ctx, hipStream_t st) {
  const size_t per = (size_t)L * hkv * hd;
  const int gx = (int)((per + 255) / 256 < 2048 ? (per + 255) / 256 : 2048);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(kv_compact_kernel<bf16_t>, dim3(gx, B), dim3(256), 0, st, (bf16_t*)kc,
                       (bf16_t*)vc, path, L, Bmax, hkv, hd, max_ctx);
  else
    hipLaunchKernelGGL(kv_compact_kernel<float>, dim3(gx, B), dim3(256), 0, st, (float*)kc,
                       (float*)vc, path, L, Bmax, hkv, hd, max_ctx);
  return hipGetLastError();
}

hipError_t launch_trace_state(const float* x, const float* ssq, int B, int n, const float* norm,
                              float eps, float* out, int ld_out, hipStream_t st) {
  if (B < 1 || n % TILE_N) return hipErrorInvalidValue;
  hipLaunchKernelGGL(trace_state_kernel, dim3(B), dim3(256), 0, st, x, ssq, B, n, norm, eps, out,
                     ld_out);
  return hipGetLastError();
}

hipError_t launch_copy_rows(void* dst, int ld_dst, const void* src, int ld_src, int rows, int cols,
                            hipStream_t st) {
  if (rows < 1 || cols < 1) return hipSuccess;
  const int gx = (cols + 255) / 256 < 64 ? (cols + 255) / 256 : 64;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(gx, rows), dim3(256), 0, st, (uint32_t*)dst, ld_dst,
                     (const uint32_t*)src, ld_src, cols);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

}  // namespace specdec
