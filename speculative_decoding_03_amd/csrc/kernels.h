// Internal launcher interface between the C-ABI layer (specdec.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

enum DType { DT_F32 = 0, DT_BF16 = 1 };
enum Epi {
  EPI_STORE = 0,
  EPI_ROPE = 1,
  EPI_SILU = 2,
  EPI_ARGMAX = 3,
  // grouped (mixture-of-experts) variants: a stacked weight of groups of tiles_per_group tiles,
  // only the listed groups computed, rows gathered and scattered through per-group row maps
  EPI_SILU_G = 4,
  EPI_STORE_G = 5
};

// One skinny GEMM  Y[M][N] = X[M][Kd] . W[N][Kd]^T  over packed tiles, with a fused
// X prologue and output epilogue.  Work unit = NU consecutive 16-row tiles (or a tile
// listed in unit_tile).  A workgroup of NW waves holds NW/KW units; each unit's reduction is
// split over KW waves and summed through LDS.  KW is fixed by (N, Kd) only.
struct GemmArgs {
  int nu = 1;  // tiles per work unit (the kernel instantiation)
  // weights
  const void* W = nullptr;
  int nkb = 0;        // Kd / 32
  int n_tiles = 0;    // tiles of the (stacked) matrix that exist
  int n_units = 0;    // launch upper bound of work units
  const int* unit_tile = nullptr;  // optional first tile of unit u
  const int* unit_row = nullptr;   // optional: argmax keeps only this row of unit u
  const int* n_units_dev = nullptr;  // optional device count of valid units
  int KW = 1, NW = 8, kb_per_split = 0;
  // weights read again soon that fit in the last-level cache (the drafter's): plain loads;
  // otherwise (the target's, streamed once per step) non-temporal loads
  int w_cached = 0;
  // weights in the 4-bit block format (common.h): bf16 activations only, nkb % 4 == 0
  int wq4 = 0;
  int M = 0;
  // grouped launches (EPI_*_G): unit u computes group g = group_list[u / units_per_group]
  // (n_groups_dev[0] groups are listed), tiles g*tiles_per_group + (u % units_per_group)*NU.
  // Local row m < M of group g reads X row xrow_map[g*M + m] (-1: empty row) and writes output
  // row orow_map[g*M + m] (-1: skipped); EPI_STORE_G scales by orow_wt[g*M + m].
  const int* group_list = nullptr;
  const int* n_groups_dev = nullptr;
  int units_per_group = 0;
  int tiles_per_group = 0;
  const int* xrow_map = nullptr;
  const int* orow_map = nullptr;
  const float* orow_wt = nullptr;
  // X operand: storage-typed [M][ldx], or the quad layout (x_qx, M <= 4; see qx_offset)
  const void* X = nullptr;
  int ldx = 0;
  int x_qx = 0;
  int out_qx = 0;  // xw_out / hout written in the quad layout (M <= 4)
  // optional row scale of the results (an RMSNorm folded in): y *= 1/sqrt(sum_t yssq[t][m] /
  // yscale_n + eps) over n_yssq tiles
  const float* yssq = nullptr;
  int n_yssq = 0;
  int yscale_n = 0;
  float eps = 0.f;
  int* err = nullptr;
  // EPI_STORE: out[m][col] (=|+=) y; optional per-tile sums of squares of the result and the
  // result times the next norm's weight in the storage type (xw_out[m][col], ld = ldo)
  float* out = nullptr;
  int ldo = 0;
  int accumulate = 0;
  float* ssq = nullptr;        // [n_tiles][ld_ssq]
  // row strides of ssq and yssq (0: M); a launch over a slice of a longer call's rows uses the
  // call's row count
  int ld_ssq = 0, ld_yssq = 0;
  // prompt GEMM (launch_mm) with its reduction split over kpart_n workgroups per block: fp32
  // partial blocks in kpart (launch_mm_partial_floats), summed in split order by a second launch
  float* kpart = nullptr;
  int kpart_n = 1;
  // optional addend rows: y = (sum_{k < add_n} addend[(m*add_n + k)*ldo + col]) + y, k ascending
  const float* addend = nullptr;
  int add_n = 0;
  void* xw_out = nullptr;
  const float* xw_norm = nullptr;
  // EPI_ROPE: columns are heads of hd with rotary pairs interleaved; heads [0,hq) -> qout,
  // [hq, hq+hkv) -> kcache, [hq+hkv, hq+2hkv) -> vcache at position len[b] + row + pos_off.
  void* qout = nullptr;  // storage-typed [M][hq][hd] (the attention's MFMA operand)
  void* kcache = nullptr;
  void* vcache = nullptr;
  const int* len = nullptr;
  int rows_per_seq = 1;
  int pos_off = 0;
  int hq = 0, hkv = 0, hd = 0;
  int max_ctx = 0;
  int cache_b_stride = 0;  // elements between sequences in one layer's cache = hkv*max_ctx*hd
  float theta = 10000.f;
  const float2* rope_cs = nullptr;  // EPI_ROPE: [max_ctx][hd/2] (cos, sin) (launch_rope_table)
  // EPI_ROPE positions of row r of a sequence: POS_LINEAR len + r + pos_off (rotary angle and
  // cache slot); POS_FLAT len + pos_off for every row (the drafter's branches, no cache write);
  // POS_TREE angle at len + tree_depth[r], cache slot len + r (a tree verify's nodes)
  int pos_mode = 0;
  const uint8_t* tree_depth = nullptr;  // POS_TREE: [rows per sequence] device (launch_tree_desc)
  // EPI_SILU: hout[m][f] = silu(gate) * up, gate/up tiles interleaved
  void* hout = nullptr;
  int ldh = 0;
  // EPI_ARGMAX: per unit (value, index) of the row maximum, lowest index on ties
  float* amax_val = nullptr;
  int* amax_idx = nullptr;
  int ld_amax = 0;
  const int* idx_map = nullptr;  // optional column -> reported index
  float* logits = nullptr;       // optional full fp32 output [M][ld_logits]
  int ld_logits = 0;
};

// Optional events attached to the kernel's own dispatch (start and end of its execution on the
// device, without the gaps between launches).
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_gemm(int dtype, int MT, int NU, int epi, const GemmArgs& a, hipStream_t st,
                       const LaunchTiming* tm = nullptr);

// Compute-bound GEMM of a prompt chunk (gemm_mm.hip): bf16 weights in the packed tile layout
// (or, with wq4, 4-bit blocks expanded to bf16 as they are staged; nkb % 4 == 0),
// row-major bf16 X of a.M rows (any count), nkb % 2 == 0; epilogues EPI_STORE, EPI_ROPE (one
// sequence: rows at positions len[0] + pos_off + row), EPI_SILU and EPI_ARGMAX (units of 64
// columns, slot row * ld_amax + unit) as in launch_gemm.  The unit fields (nu, n_units, KW, NW,
// kb_per_split) are not used.  With kpart_n > 1 the reduction is split
// kpart_n ways over 256 x 256 blocks into a.kpart, which holds launch_mm_partial_floats floats.
hipError_t launch_mm(int epi, const GemmArgs& a, hipStream_t st, const LaunchTiming* tm = nullptr);
size_t launch_mm_partial_floats(int n_tiles, int M, int kpart_n);

// The 4-bit block weight format (common.h): a matrix [N][Kd] with N % 16 == 0 and
// Kd % 128 == 0 takes q4_bytes(N, Kd) bytes.  launch_pack_q4 writes it from codes [N][Kd] (one
// byte each, 0..15) and fp16 steps [N][Kd / 32], rows permuted by `kind` as launch_pack does.
__host__ __device__ inline size_t q4_bytes(size_t N, size_t Kd) { return N * Kd / 2 + N * (Kd / 32) * 2; }
hipError_t launch_pack_q4(const uint8_t* q, const uint16_t* steps, void* dst, int N, int Kd,
                          int kind, int hd, int split_rows, hipStream_t st);

// Grouped-query attention of R query rows per sequence over one layer's cache: K [pos][hd],
// V transposed [hd][pos].
// Row i of sequence b sees keys [0, len[b] + i + key_off).  Chunks of CH keys at fixed absolute
// positions leave (max, sum of exponentials, value sum) partials that a second kernel combines
// in chunk order.
struct AttnArgs {
  const void* q = nullptr;  // storage-typed [B*R][hq][hd]
  const void* kcache = nullptr;
  const void* vcache = nullptr;
  const int* len = nullptr;
  void* out = nullptr;  // storage-typed [B*R][hq*hd], row-major or the quad layout (out_qx)
  int out_qx = 0;
  float* part = nullptr;
  int* err = nullptr;
  int B = 0, R = 0, key_off = 0;
  int hq = 0, hkv = 0, hd = 0;
  int max_ctx = 0;
  int cache_b_stride = 0;
  int chunk = 256;
  int n_chunks = 0;  // chunks per head in the partial buffer = ceil(max_ctx / chunk)
  int n_launch = 0;  // chunks launched: covers the host-side bound on the keys any row sees
  float scale = 0.f;
  // Keys row i of a sequence sees: VIS_CAUSAL [0, len + i + key_off) (verify rows, the drafter's
  // single row); VIS_FLAT [0, len + key_off) for every row (the drafter's branches of a tree
  // draft); VIS_TREE [0, len) and slot len + j for every bit j of tree_mask[i] (a tree verify:
  // node i sees its ancestors and itself, each at slot len + node index).
  int vis = 0;
  const uint64_t* tree_mask = nullptr;  // VIS_TREE: [R] device (launch_tree_desc)
  // 1: each workgroup takes one 16-vector tile of the query vectors instead of all of them (more
  // workgroups for launches that would not fill the chip; every vector's arithmetic is unchanged)
  int q_split = 0;
};
enum { VIS_CAUSAL = 0, VIS_FLAT = 1, VIS_TREE = 2 };
enum { POS_LINEAR = 0, POS_FLAT = 1, POS_TREE = 2 };

// Keys [0, end) hold every key some row of the call may see.
__host__ __device__ inline int attn_key_end(int vis, int len, int R, int key_off) {
  return vis == VIS_FLAT ? len + key_off : (vis == VIS_TREE ? len + R : len + R - 1 + key_off);
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st);
// The rows of a prompt chunk of one sequence (B = 1, VIS_CAUSAL, bf16, head size 64, 128 or
// 256): every row's attention over the committed prefix and the chunk, written to out
// (row-major).  n_chunks <= 1: each workgroup walks all keys of its query vectors; n_chunks > 1
// (= n_launch): the keys split into ranges of `chunk` keys (a multiple of 64, chunk * n_chunks
// covering every key a row sees), partials in part ([hkv][n_chunks][R*hq/hkv][hd + 4] floats)
// merged by the combine.
hipError_t launch_attention_prompt(const AttnArgs& a, hipStream_t st);
int attention_prompt_nwq(int R, int hq, int hkv);    // waves per prompt-attention workgroup
int attention_prompt_block(int R, int hq, int hkv);  // query vectors per workgroup
int attention_chunk(int n_kv_heads, int max_ctx);  // keys per chunk (fixed per model and context)
// whether a launch of n_launch chunks x hkv heads x B sequences of R rows x G query heads splits
// its query tiles over workgroups (AttnArgs::q_split)
bool attention_q_split(int n_launch, int hkv, int B, int R, int G);
bool attention_supported(int head_dim);     // head sizes the attention kernel is built for

// Misc kernels (misc.hip).
hipError_t launch_embed(int dtype, const void* E, int nkb, int d, const int* tokens, int M,
                        float* x, float* ssq, void* xw, int xw_qx, const float* norm, int vocab,
                        int* err, hipStream_t st, int e_q4 = 0);
hipError_t launch_accept(const float* amax_val, const int* amax_idx, int n_parts, int ld_amax,
                         int B, int R, const int* tokens, int* out_tokens, int* n_emit,
                         int* next_tok, int commit, int* len, float* hid, const float* X, int d,
                         int* argmax_out, int* err, hipStream_t st);
// Prompt prefill (misc.hip): per-row argmax over LM-head partials [rows][ld]; commit of n rows
// of one sequence (len += n, hid = the last row).
hipError_t launch_rows_argmax(const float* amax_val, const int* amax_idx, int n_parts, int ld,
                              int rows, int* out, hipStream_t st);
hipError_t launch_commit_rows(int* len, float* hid, const float* xlast, int d, int n,
                              hipStream_t st);
hipError_t launch_commit(const int* n_commit, int B, int R, int* len, float* hid, const float* X,
                         int d, int* err, hipStream_t st);
hipError_t launch_draft_input(int dtype, const float* h, const int* tok, const void* table,
                              int nkb_table, const int* vocab_row, int vocab, const float* norm_h,
                              const float* norm_e, int d, int Dd, float eps, void* u, int u_qx,
                              int B, int* err, hipStream_t st, int h_div = 1, int t_q4 = 0);
// Tree drafts (misc.hip): the first level's top-w tokens, the later levels' per-branch tokens,
// the acceptance walk over a tree and the compaction of the accepted path's cache entries.
hipError_t launch_tree_top(const float* scores, int vocab, const int* unit_tile, int units_per_seq,
                           int rows_per_unit, const int* row_vocab, int B, int w, int D,
                           const int* cur_tok, const int* len, const int* inject, int inj_stride,
                           int* tree_tok, int* raw, int* err, hipStream_t st);
hipError_t launch_tree_finalize(const float* amax_val, const int* amax_idx, int ld_amax, int parts,
                                int seq_offset, int rows, int w, int D, int depth, const int* len,
                                const int* inject, int inj_stride, int* tree_tok, int* raw,
                                int* err, hipStream_t st);
hipError_t launch_tree_accept(const float* amax_val, const int* amax_idx, int n_parts, int ld_amax,
                              int B, int n_nodes, const int8_t* parent, const int* tokens,
                              int* out_tokens, int out_ld, int* n_emit, int* next_tok, int commit,
                              int* len, float* hid, const float* X, int d, int* path, int* err,
                              hipStream_t st);
// Writes a tree's per-node visibility masks (uint64 [n]) and depths (uint8 [n]) to device memory
// for the verify's attention and rotary epilogue.
hipError_t launch_tree_desc(int n, const uint64_t* mask, const uint8_t* depth, uint64_t* mask_out,
                            uint8_t* depth_out, hipStream_t st);
hipError_t launch_kv_compact(int dtype, void* kc, void* vc, const int* path, int L, int B,
                             int Bmax, int hkv, int hd, int max_ctx, hipStream_t st);
// Mixture-of-experts routing of M rows over E experts (logits [M][E]): the top_k experts of
// each row (ties -> lower id), softmax weights over them, and the per-expert row maps of the
// grouped GEMMs: for expert e and its i-th routed row m (ascending m), xrow[e*M+i] = m,
// orow[e*M+i] = m*top_k + r (r = rank of e among the row's experts in ascending id) and
// wt[e*M+i] = its weight; -1 beyond the expert's count.  group_list = experts with at least one
// row, ascending, n_groups[0] of them.  usage (optional): += n_groups.
hipError_t launch_moe_route(const float* logits, int M, int E, int top_k, int* xrow, int* orow,
                            float* wt, int* group_list, int* n_groups, int* usage, int* err,
                            hipStream_t st);
hipError_t launch_cluster_select(const float* z, int Nc, int k_c, int B, int tiles_per_cluster,
                                 int units_per_cluster, int* unit_tile, int* unit_row, int* err,
                                 hipStream_t st);
hipError_t launch_draft_finalize(const float* amax_val, const int* amax_idx, int ld_amax,
                                 int parts_per_seq, int seq_offset, int B, int K, int j,
                                 const int* len,
                                 const int* inject, int inj_stride, int* drafts, int* dtok,
                                 const int* cur_tok, int* vtok, int* err, hipStream_t st);
// Drafter trace helpers (tests and measurement): s[b] = x[b] * rs(b) * norm into out[b*ld_out],
// rs(b) = 1/sqrt(sum_t ssq[t][b] / n + eps) over n/16 tiles (the row scale the head's epilogue
// forms); and a strided copy of rows of 32-bit words.
hipError_t launch_trace_state(const float* x, const float* ssq, int B, int n, const float* norm,
                              float eps, float* out, int ld_out, hipStream_t st);
hipError_t launch_copy_rows(void* dst, int ld_dst, const void* src, int ld_src, int rows, int cols,
                            hipStream_t st);
hipError_t launch_pack(int dtype, const void* src, void* dst, int N, int Kd, int kind, int hd,
                       int split_rows, hipStream_t st);
hipError_t launch_fill_i32(int* p, int v, size_t n, hipStream_t st);
// t[pos][i] = (cos, sin) of pos * theta^(-2i/hd), pos < max_ctx, i < hd/2.
hipError_t launch_rope_table(float2* t, int hd, int max_ctx, float theta, hipStream_t st);

}  // namespace specdec
