// C-ABI layer of libspecdec: validation, workspace carving, the per-shape work split of every
// projection, and the launch sequences of draft / verify / accept / commit.  All device memory
// belongs to the caller; nothing here allocates, frees or synchronises on the step path.

#include "../../include/specdec.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"

using namespace specdec;

// Workspace of contexts made by specdec_create_static (callers that cannot allocate device
// memory): one fixed array per GPU, held by the loaded library until the process ends.  Host
// code never uses this name as an address: the per-device address comes from
// hipGetSymbolAddress (static_workspace below).
static __device__ __align__(256) unsigned char scratch[SPECDEC_STATIC_WORKSPACE_BYTES];

namespace {

constexpr size_t ALIGN = 256;
constexpr int TARGET_WAVES = 2048;   // waves per projection launch
constexpr int MIN_KB_PER_WAVE = 8;   // k-blocks each wave streams at least
// ... and in projections of fewer than SMALL_UNITS units (measured on MI355X at the E2B shapes:
// q/k/v 7.8 -> 6.6 us, o + down 14.1 -> 13.3 us, verify 1.164 -> 1.137 ms, draft 0.438 -> 0.425 ms)
constexpr int MIN_KB_PER_WAVE_SMALL = 4;
constexpr int SMALL_UNITS = 256;
// ... and in the argmax projections (the LM head: measured on MI355X, E2B 146.7 -> 131.7 us with
// one wave over all 48 k-blocks instead of four, E4B 235.3 -> 224.9 us with two instead of eight,
// 31B 412.9 -> 407.5 us with four instead of eight)
constexpr int MIN_KB_PER_WAVE_ARGMAX = 40;
constexpr int WIDE_NU = 8;            // tiles per gated unit in calls of 17..32 rows
constexpr int MM_SPLIT_WGS = 240;     // workgroups of a prompt GEMM whose reduction is split
// prompt attention: workgroups the key ranges aim at, and the most ranges (measured on MI355X,
// 512-row prompts: 512 workgroups are 4% slower at the 31B shape, 2048 and 8 ranges no faster)
constexpr int PROMPT_ATTN_WGS = 1024;
constexpr int PROMPT_MAX_RANGES = 4;
constexpr int PROMPT_SPLIT_KEYS = 1024;
constexpr int WIDE_MIN_UNITS = 400;   // ... when that leaves at least this many units
constexpr int WIDE4_MIN_UNITS = 128;  // else units of four tiles when that leaves this many
// 4-bit weights carry 3.6x fewer bytes per k-block: each wave streams at least 16 (measured on
// MI355X at the 31B shapes: 16 beats 8 and 32; wide gated projections split at most 4 ways)
constexpr int MIN_KB_PER_WAVE_Q4 = 16;
constexpr int GATED_MAX_KW_Q4 = 4;
// Tiles per unit of the target's q/k/v, o and down projections: two when the projection has at
// least 256 tiles (one activation load then serves twice the weight bytes), else one, which keeps
// more workgroups on the CUs (measured on MI355X: two at the 31B shapes, one at the E2B, E4B and
// MoE model widths).
int store_nu(int N) { return N / 16 >= 256 ? 2 : 1; }

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int cdiv(int a, int b) { return (a + b - 1) / b; }

// k-blocks per split rounded up to whole quad blocks (four k-blocks), so that every split of an
// operand in the quad layout starts on a block
int round_up4(int v) { return (v + 3) / 4 * 4; }

int pow2_floor(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

// One projection: packed weights plus its fixed work split (a function of N and Kd only).
struct Gemm {
  const void* W = nullptr;
  int N = 0, Kd = 0, nkb = 0, n_tiles = 0, NU = 1, n_units = 0, KW = 1, NW = 8, kbps = 0;
  int tpg = 0, upg = 0;  // grouped (stacked experts): tiles and units per group
  int nu_wide = 0;       // tiles per unit for calls of 17..32 rows (0: NU)
  bool cached = false;   // the drafter's weights: re-read every sub-step, kept in the caches
};

// Split-K factor of a projection with `units` work units of NU tiles over nkb k-blocks.  Measured
// on MI355X at the 31B shapes (M = 4): about TARGET_WAVES waves per launch, each streaming at
// least MIN_KB_PER_WAVE k-blocks (MIN_KB_PER_WAVE_SMALL in small projections), is best for
// one-tile units; the 4-tile argmax units (LM head, drafter table) of bf16 weights stream best
// with at least MIN_KB_PER_WAVE_ARGMAX k-blocks per wave, split at most 8 ways.
int split_for(int units, int nkb, int NU, bool q4) {
  const int mkb = q4 ? MIN_KB_PER_WAVE_Q4
                     : (NU >= 4 ? MIN_KB_PER_WAVE_ARGMAX
                                : (units < SMALL_UNITS ? MIN_KB_PER_WAVE_SMALL : MIN_KB_PER_WAVE));
  int KW = NU >= 4 ? 8 : cdiv(TARGET_WAVES, units);
  KW = std::min({KW, 16, std::max(1, nkb / mkb)});
  return pow2_floor(std::max(1, KW));
}

// Waves per workgroup for a split-K factor KW (a workgroup holds NW / KW whole units).
int waves_for(int KW) { return KW == 16 ? 16 : 8; }

Gemm make_gemm(const void* W, int N, int Kd, int NU, bool q4, bool allow_split = true,
               bool gated = false) {
  Gemm g;
  g.W = W;
  g.N = N;
  g.Kd = Kd;
  g.nkb = Kd / 32;
  g.n_tiles = N / 16;
  g.NU = NU;
  g.n_units = cdiv(g.n_tiles, NU);
  g.KW = allow_split ? split_for(g.n_units, g.nkb, NU, q4) : 1;
  g.NW = waves_for(g.KW);
  if (allow_split && gated && g.n_units >= 4 * TARGET_WAVES / 8) {
    // wide gated projections: one unit per workgroup, split up to eight ways (measured on
    // MI355X at the 31B gate/up shape: the small workgroups balance over the CUs as they
    // retire, and eight waves keep more loads in flight than four)
    g.KW = std::min(q4 ? GATED_MAX_KW_Q4 : 8,
                    std::max(1, pow2_floor(g.nkb / (q4 ? MIN_KB_PER_WAVE_Q4 : MIN_KB_PER_WAVE))));
    g.NW = std::max(4, g.KW);
  }
  g.kbps = round_up4(cdiv(g.nkb, g.KW));
  if (gated && !q4 && NU == 2 && g.n_tiles % WIDE_NU == 0 && g.n_tiles / WIDE_NU >= WIDE_MIN_UNITS)
    g.nu_wide = WIDE_NU;
  else if (gated && !q4 && NU == 2 && g.n_tiles % 4 == 0 && g.n_tiles / 4 >= WIDE4_MIN_UNITS)
    g.nu_wide = 4;
  return g;
}

// M-tiles (16 rows each) of a call of M rows
int mt_for(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// Calls of 17..32 rows (two M-tiles) read two activation fragments per k-block for every unit,
// as many bytes as the unit's two weight tiles.  A wide gated projection then takes units of
// WIDE_NU tiles (four gate/up pairs), which share each activation load over four times the
// weight bytes.  The split-K stays the same, so each column's sum is formed in the same order
// as in any other call, and each workgroup takes one unit.  Measured on MI355X at 32 rows: the
// 31B gate/up 154 -> 123 us (units of four tiles: 128 us); the MoE shared FFN's gate/up (704
// tiles, too few for 8-tile units) with 4-tile units 27.6 -> 24.1 us (35.7 us with two units per
// 8-wave workgroup).  At 16 rows and fewer the two-tile units are faster.
void wide_units(GemmArgs& a, const Gemm& g, int M) {
  if (g.nu_wide && mt_for(M) == 2) {
    a.nu = g.nu_wide;
    a.n_units = g.n_tiles / g.nu_wide;
    a.NW = std::max(4, g.KW);
  }
}

// A stacked weight of E groups (experts) of N x Kd each, of which a launch computes only the
// routed ones.  The split is sized for the top_k groups of one row, fixed per shape so that a
// row's result does not depend on how many other rows share the launch.
Gemm make_grouped_gemm(const void* W, int N, int Kd, int NU, int E, int top_k, bool q4) {
  Gemm g;
  g.W = W;
  g.N = N;
  g.Kd = Kd;
  g.nkb = Kd / 32;
  g.tpg = N / 16;
  g.upg = g.tpg / NU;
  g.n_tiles = E * g.tpg;
  g.NU = NU;
  g.n_units = E * g.upg;
  g.KW = split_for(top_k * g.upg, g.nkb, NU, q4);
  g.NW = waves_for(g.KW);
  g.kbps = round_up4(cdiv(g.nkb, g.KW));
  return g;
}

struct Layout {
  size_t x, xw, q, o, h, ssq, ssq_d, amax_v, amax_i, att_part, err, rope;
  size_t rlog, e_xrow, e_orow, e_wt, e_groups, e_ngroups, e_h, e_y, e_usage;
  size_t u, xd, xdw, dh, hnext, z, utile, urow, dtok, d_amax_v, d_amax_i, tscore, path;
  size_t tree_mask, tree_depth;
  // prompt prefill (max_prefill rows): activations, argmax partials and attention partials
  size_t p_x, p_xw, p_ssq, p_q, p_o, p_h, p_amax_v, p_amax_i, p_part;
  size_t total;
};

struct Dims {
  int Mx, Bx, Rall_max, n_chunks, chunk, esz, parts;
};

}  // namespace

struct specdec_ctx {
  specdec_config cfg{};
  Dims dm{};
  Layout lay{};
  char* ws = nullptr;
  void* kv_k = nullptr;
  void* kv_v = nullptr;
  int* len = nullptr;
  float* hid = nullptr;
  std::vector<const void*> lw, dw;
  specdec_weights w{};
  std::vector<Gemm> g_qkv, g_o, g_gu, g_down;
  std::vector<Gemm> g_router, g_egu, g_edown;  // mixture of experts
  Gemm g_head, g_in, g_back, g_cent, g_table, g_clu;
  std::vector<Gemm> g_dq, g_do, g_dgu, g_ddown;
  std::vector<int> len_hi;  // host-side upper bound on len
  int last_B = 0, last_R = 0;
  int last_tree_n = 0;           // node count of the last tree verify (0: a linear verify)
  int8_t last_parent[64] = {};   // its shape
  int prof_class = -1, prof_cap = 0, prof_n = 0;
  bool moe_usage_on = false;
  std::vector<hipEvent_t> prof_ev;
};

namespace {

// Width of the dense gated FFN: the FFN itself, or the shared FFN of a mixture-of-experts layer.
int ffn_width(const specdec_config* c) { return c->n_experts > 0 ? c->shared_ffn : c->ffn_dim; }

bool valid_config(const specdec_config* c) {
  if (!c) return false;
  if (c->n_experts < 0) return false;
  if (c->n_experts > 0) {
    if (c->n_experts > 256 || c->n_experts % 16 || c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return false;
    if (c->expert_ffn % 32 || c->expert_ffn < 32 || c->shared_ffn % 32 || c->shared_ffn < 32)
      return false;
  }
  if (c->dtype != SPECDEC_F32 && c->dtype != SPECDEC_BF16) return false;
  if (c->weight_format != SPECDEC_WF_DENSE && c->weight_format != SPECDEC_WF_Q4) return false;
  if (c->weight_format == SPECDEC_WF_Q4) {
    // 4-bit blocks: bf16 activations, whole 128-element k-groups on every reduction axis
    const int qd = c->n_q_heads * c->head_dim;
    if (c->dtype != SPECDEC_BF16) return false;
    for (int k : {c->d_model, qd, c->n_experts > 0 ? c->shared_ffn : c->ffn_dim, c->d_dim, c->d_ffn})
      if (k % 128) return false;
    if (c->n_experts > 0 && c->expert_ffn % 128) return false;
  }
  if (c->n_layers < 1 || c->d_model < 32 || c->n_q_heads < 1 || c->n_kv_heads < 1) return false;
  if (c->n_q_heads % c->n_kv_heads) return false;
  if (c->head_dim % 16 || c->head_dim > 256 || c->head_dim < 16) return false;
  const int qd = c->n_q_heads * c->head_dim;
  if (c->d_model % 32 || qd % 32) return false;
  if (c->n_experts == 0 && (c->ffn_dim % 32 || c->ffn_dim < 32)) return false;
  if (c->d_layers < 1 || c->d_dim % 32 || c->d_dim < 32 || c->d_dim > 1024) return false;
  if (c->d_ffn % 32 || c->d_ffn < 32) return false;
  if (c->vocab % 64 || c->vocab < 64 || c->n_centroids < 16 || c->n_centroids % 16) return false;
  if (c->vocab % c->n_centroids || (c->vocab / c->n_centroids) % 64) return false;
  if (c->max_batch < 1 || c->max_rows < 1 || c->max_rows > 64) return false;
  if (c->max_batch * c->max_rows > 64) return false;
  if (c->max_draft < 1 || c->max_draft + 1 > c->max_rows) return false;
  if (c->max_ctx < c->max_rows + 1 || c->max_ctx > (1 << 20) || c->max_ctx % 8) return false;
  if (c->max_ctx / attention_chunk(c->n_kv_heads, c->max_ctx) > 4096) return false;
  if (c->max_prefill < 0 || c->max_prefill > 1024) return false;
  if (c->max_prefill > 0) {
    // the prompt GEMM: bf16 weights of a dense model, reduction widths in stages of 64
    const int qd = c->n_q_heads * c->head_dim;
    if (c->dtype != SPECDEC_BF16 || c->n_experts > 0) return false;
    if (c->d_model % 64 || qd % 64 || c->ffn_dim % 64) return false;
    // the prompt attention's head sizes
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return false;
  }
  if (c->kv_src_layer >= c->n_layers) return false;
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return false;
  return true;
}

Dims make_dims(const specdec_config* c) {
  Dims d;
  d.Bx = c->max_batch;
  d.Mx = c->max_batch * c->max_rows;
  d.Rall_max = c->max_rows * (c->n_q_heads / c->n_kv_heads);
  d.chunk = attention_chunk(c->n_kv_heads, c->max_ctx);
  d.n_chunks = cdiv(c->max_ctx, d.chunk);
  d.esz = c->dtype == SPECDEC_BF16 ? 2 : 4;
  d.parts = c->vocab / 64;
  return d;
}

Layout make_layout(const specdec_config* c, const Dims& dm) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 4));
    return o;
  };
  const int d = c->d_model, qd = c->n_q_heads * c->head_dim, Dd = c->d_dim;
  L.x = take((size_t)dm.Mx * d * 4);
  // GEMM operands (row-major [rows][K], or the quad layout when a call has at most 4 rows)
  auto xbuf = [&](size_t K) { return take((size_t)std::max(dm.Mx, 4) * ((K + 127) / 128 * 128) * dm.esz); };
  L.xw = xbuf(d);
  L.q = take((size_t)dm.Mx * qd * 4);
  L.o = xbuf(qd);
  L.h = xbuf(ffn_width(c));
  L.ssq = take((size_t)dm.Mx * (d / 16) * 4);
  L.ssq_d = take((size_t)dm.Mx * (Dd / 16) * 4);  // drafter rows: sequences x tree branches
  L.amax_v = take((size_t)dm.Mx * dm.parts * 4);
  L.amax_i = take((size_t)dm.Mx * dm.parts * 4);
  // attention chunk partials: per (sequence, kv head, chunk) Rall rows of (o[hd], m, l, 2 pad)
  L.att_part = take((size_t)dm.Bx * c->n_kv_heads * dm.n_chunks * dm.Rall_max * (c->head_dim + 4) * 4);
  L.err = take(64);
  L.rope = take((size_t)c->max_ctx * (c->head_dim / 2) * 8);
  L.u = xbuf(d + Dd);
  L.xd = take((size_t)dm.Mx * Dd * 4);
  L.xdw = xbuf(Dd);
  L.dh = xbuf(c->d_ffn);
  L.hnext = take((size_t)dm.Mx * d * 4);
  L.z = take((size_t)dm.Mx * c->n_centroids * 4);
  L.utile = take((size_t)dm.Mx * dm.parts * 4);
  L.urow = take((size_t)dm.Mx * dm.parts * 4);
  L.dtok = take((size_t)dm.Mx * 4);
  L.d_amax_v = take((size_t)dm.Mx * dm.parts * 4);  // [rows][V/64] (full) or [rows*k_c*upc] (clustered)
  L.d_amax_i = take((size_t)dm.Mx * dm.parts * 4);
  L.tscore = take((size_t)dm.Bx * c->vocab * 4);  // a tree draft's first-level scores, by table row
  L.path = take((size_t)dm.Bx * 65 * 4);         // accepted tree paths for the cache compaction
  L.tree_mask = take(64 * 8);                     // the verified tree: visibility masks
  L.tree_depth = take(64);                        // and node depths
  const size_t E = c->n_experts, slots = (size_t)dm.Mx * c->top_k;
  L.rlog = take((size_t)dm.Mx * E * 4);
  L.e_xrow = take(E * dm.Mx * 4);
  L.e_orow = take(E * dm.Mx * 4);
  L.e_wt = take(E * dm.Mx * 4);
  L.e_groups = take(E * 4);
  L.e_ngroups = take(4);
  L.e_h = take(slots * c->expert_ffn * dm.esz);
  L.e_y = take(slots * d * 4);
  L.e_usage = take((size_t)c->n_layers * 4);  // experts routed to, summed per layer (measurement)
  const size_t P = (size_t)c->max_prefill;
  if (P > 0) {
    L.p_x = take(P * d * 4);
    L.p_xw = take(P * d * 2);
    L.p_ssq = take(P * (d / 16) * 4);
    L.p_q = take(P * qd * 2);
    L.p_o = take(P * qd * 2);
    L.p_h = take(P * c->ffn_dim * 2);
    L.p_amax_v = take(P * dm.parts * 4);
    L.p_amax_i = take(P * dm.parts * 4);
    // the prompt GEMM's split partial blocks (at most MM_SPLIT_WGS blocks of one split launch)
    // and, at other times of the layer, the prompt attention's key-range partials
    const size_t G = (size_t)(c->n_q_heads / c->n_kv_heads);
    L.p_part = take(std::max(launch_mm_partial_floats(16, 256, MM_SPLIT_WGS) * 4,
                             (size_t)c->n_kv_heads * PROMPT_MAX_RANGES * P * G * (c->head_dim + 4) * 4));
  }
  L.total = off;
  return L;
}

void build_gemms(specdec_ctx* x) {
  const specdec_config& c = x->cfg;
  const int d = c.d_model, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const int Fw = ffn_width(&c);
  const bool q4 = c.weight_format == SPECDEC_WF_Q4;
  x->g_qkv.clear(); x->g_o.clear(); x->g_gu.clear(); x->g_down.clear();
  x->g_router.clear(); x->g_egu.clear(); x->g_edown.clear();
  x->g_dq.clear(); x->g_do.clear(); x->g_dgu.clear(); x->g_ddown.clear();
  for (int l = 0; l < c.n_layers; ++l) {
    const void* const* t = x->lw.data() + (size_t)l * SPECDEC_N_LAYER_TENSORS;
    x->g_qkv.push_back(make_gemm(t[SPECDEC_LW_QKV], qd + 2 * kvd, d, store_nu(qd + 2 * kvd), q4));
    x->g_o.push_back(make_gemm(t[SPECDEC_LW_O], d, qd, store_nu(d), q4));
    x->g_gu.push_back(make_gemm(t[SPECDEC_LW_GATE_UP], 2 * Fw, d, 2, q4, true, true));
    if (c.dtype != SPECDEC_BF16) x->g_gu.back().nu_wide = 0;  // wide units: bf16 only
    x->g_down.push_back(make_gemm(t[SPECDEC_LW_DOWN], d, Fw, store_nu(d), q4));
    if (c.n_experts > 0) {
      x->g_router.push_back(make_gemm(t[SPECDEC_LW_ROUTER], c.n_experts, d, 1, q4));
      x->g_egu.push_back(make_grouped_gemm(t[SPECDEC_LW_EXP_GATE_UP], 2 * c.expert_ffn, d, 2,
                                           c.n_experts, c.top_k, q4));
      x->g_edown.push_back(make_grouped_gemm(t[SPECDEC_LW_EXP_DOWN], d, c.expert_ffn, 1,
                                             c.n_experts, c.top_k, q4));
    }
  }
  x->g_head = make_gemm(x->w.embed, c.vocab, d, 4, q4);
  x->g_in = make_gemm(x->w.w_in, c.d_dim, d + c.d_dim, 1, q4);
  x->g_back = make_gemm(x->w.w_back, d, c.d_dim, 1, q4);
  x->g_cent = make_gemm(x->w.centroids, c.n_centroids, c.d_dim, 1, q4);
  x->g_table = make_gemm(x->w.table, c.vocab, c.d_dim, 4, q4);
  x->g_clu = make_gemm(x->w.table, c.vocab, c.d_dim, 4, q4, false);
  for (int l = 0; l < c.d_layers; ++l) {
    const void* const* t = x->dw.data() + (size_t)l * SPECDEC_N_DRAFT_TENSORS;
    x->g_dq.push_back(make_gemm(t[SPECDEC_DW_Q], qd, c.d_dim, 1, q4));
    x->g_do.push_back(make_gemm(t[SPECDEC_DW_O], c.d_dim, qd, 1, q4));
    x->g_dgu.push_back(make_gemm(t[SPECDEC_DW_GATE_UP], 2 * c.d_ffn, c.d_dim, 2, q4, true, true));
    x->g_ddown.push_back(make_gemm(t[SPECDEC_DW_DOWN], c.d_dim, c.d_ffn, 1, q4));
  }
  // the drafter's weights (about 170 MB at the 31B shape, the full table included) are read
  // again in every sub-step and fit in the 256 MB last-level cache
  for (Gemm* g : {&x->g_in, &x->g_back, &x->g_cent, &x->g_table, &x->g_clu}) g->cached = true;
  for (auto* v : {&x->g_dq, &x->g_do, &x->g_dgu, &x->g_ddown})
    for (Gemm& g : *v) g.cached = true;
}

template <typename P>
P* at(specdec_ctx* x, size_t off) {
  return reinterpret_cast<P*>(x->ws + off);
}


int dt_of(const specdec_ctx* x) { return x->cfg.dtype == SPECDEC_BF16 ? DT_BF16 : DT_F32; }

// Times one launch of the profiled class.  A single-kernel launch takes the events attached to
// its own dispatch (timing()); otherwise the scope records stream events around the launches.
struct ProfScope {
  specdec_ctx* x;
  bool on, attached = false;
  hipStream_t st;
  LaunchTiming tm;
  ProfScope(specdec_ctx* c, int cls, hipStream_t s, bool single_kernel = false)
      : x(c), on(false), st(s) {
    if (cls >= 0 && x->prof_class == cls && x->prof_n < x->prof_cap) {
      on = true;
      attached = single_kernel;
      tm.start = x->prof_ev[2 * x->prof_n];
      tm.stop = x->prof_ev[2 * x->prof_n + 1];
      if (!attached) (void)hipEventRecord(tm.start, st);
    }
  }
  const LaunchTiming* timing() const { return on && attached ? &tm : nullptr; }
  ~ProfScope() {
    if (on) {
      if (!attached) (void)hipEventRecord(tm.stop, st);
      x->prof_n++;
    }
  }
};

GemmArgs base_args(specdec_ctx* x, const Gemm& g, int M) {
  GemmArgs a;
  a.W = g.W;
  a.nu = g.NU;
  a.nkb = g.nkb;
  a.n_tiles = g.n_tiles;
  a.n_units = g.n_units;
  a.KW = g.KW;
  a.NW = g.NW;
  a.kb_per_split = g.kbps;
  a.w_cached = g.cached ? 1 : 0;
  a.wq4 = x->cfg.weight_format == SPECDEC_WF_Q4;
  a.M = M;
  a.x_qx = a.out_qx = M <= 4;  // activations of calls with at most 4 rows use the quad layout
  a.err = at<int>(x, x->lay.err);
  a.eps = x->cfg.rms_eps;
  return a;
}

// Normalised input: X = x * w in the storage type (written by the producer of x), results
// scaled by the RMSNorm row scale formed from the producer's per-tile sums of squares.
void norm_input(GemmArgs& a, const void* xw, int ld, const float* ssq, int n) {
  a.X = xw;
  a.ldx = ld;
  a.yssq = ssq;
  a.n_yssq = n / 16;
  a.yscale_n = n;
}

// Residual update x (+)= y that also leaves y's sums of squares and y * w_next.
void resid_output(GemmArgs& a, float* x, int ld, int accumulate, float* ssq, void* xw,
                  const float* w_next) {
  a.out = x;
  a.ldo = ld;
  a.accumulate = accumulate;
  a.ssq = ssq;
  a.xw_out = xw;
  a.xw_norm = w_next;
}

#define HIP_TRY(expr)                               \
  do {                                              \
    if ((expr) != hipSuccess) return SPECDEC_E_HIP; \
  } while (0)

int run(specdec_ctx* x, int cls, int epi, const GemmArgs& a, hipStream_t st) {
  ProfScope ps(x, cls, st, a.n_units > 0);
  HIP_TRY(launch_gemm(dt_of(x), mt_for(a.M), a.nu, epi, a, st, ps.timing()));
  return SPECDEC_OK;
}

// Routed experts of one mixture-of-experts layer over the M rows of x * ffn_norm (XW, with the
// row scales from ssq): router logits, top-k routing, then the gate/up and down projections of
// only the routed experts over their gathered rows.  Leaves w_e * FFN_e(row) in e_y at slot
// row*top_k + rank (rank = the expert's place among the row's experts in ascending id).
int routed_experts(specdec_ctx* x, int l, int M, hipStream_t st) {
  const specdec_config& c = x->cfg;
  const int d = c.d_model, E = c.n_experts;
  void* XW = x->ws + x->lay.xw;
  float* ssq = at<float>(x, x->lay.ssq);
  int* xrow = at<int>(x, x->lay.e_xrow);
  int* orow = at<int>(x, x->lay.e_orow);
  float* wt = at<float>(x, x->lay.e_wt);
  int* groups = at<int>(x, x->lay.e_groups);
  int* ngroups = at<int>(x, x->lay.e_ngroups);
  int rc;
  {  // router logits [M][E] of the normalised rows
    GemmArgs a = base_args(x, x->g_router[l], M);
    norm_input(a, XW, d, ssq, d);
    a.out = at<float>(x, x->lay.rlog);
    a.ldo = E;
    if ((rc = run(x, -1, EPI_STORE, a, st))) return rc;
  }
  HIP_TRY(launch_moe_route(at<float>(x, x->lay.rlog), M, E, c.top_k, xrow, orow, wt, groups,
                           ngroups, x->moe_usage_on ? at<int>(x, x->lay.e_usage) + l : nullptr,
                           at<int>(x, x->lay.err), st));
  // at most min(E, M*top_k) experts are routed to
  const int max_groups = std::min(E, M * c.top_k);
  {  // gate/up of the routed experts over their rows -> SiLU product at the row's slot
    const Gemm& g = x->g_egu[l];
    GemmArgs a = base_args(x, g, M);
    a.n_units = max_groups * g.upg;
    norm_input(a, XW, d, ssq, d);
    a.group_list = groups;
    a.n_groups_dev = ngroups;
    a.units_per_group = g.upg;
    a.tiles_per_group = g.tpg;
    a.xrow_map = xrow;
    a.orow_map = orow;
    a.hout = x->ws + x->lay.e_h;  // slot rows: row-major
    a.ldh = c.expert_ffn;
    a.out_qx = 0;
    if ((rc = run(x, 7, EPI_SILU_G, a, st))) return rc;
  }
  {  // down of the routed experts, scaled by the routing weight, stored at the row's slot
    const Gemm& g = x->g_edown[l];
    GemmArgs a = base_args(x, g, M);
    a.n_units = max_groups * g.upg;
    a.X = x->ws + x->lay.e_h;
    a.ldx = c.expert_ffn;
    a.x_qx = 0;
    a.group_list = groups;
    a.n_groups_dev = ngroups;
    a.units_per_group = g.upg;
    a.tiles_per_group = g.tpg;
    a.xrow_map = orow;  // the slot rows the gate/up step wrote
    a.orow_map = orow;
    a.orow_wt = wt;
    a.out = at<float>(x, x->lay.e_y);
    a.ldo = d;
    if ((rc = run(x, 8, EPI_STORE_G, a, st))) return rc;
  }
  return SPECDEC_OK;
}

// A token tree as the kernels take it: node i (topological order, parent[0] = -1) sits at depth
// depth[i] (its rotary position is len + depth) in cache slot len + i, and sees the committed
// prefix and the slots of the nodes in mask[i] (its ancestors and itself).
struct Tree {
  int n = 0, max_depth = 0;
  int8_t parent[64] = {};
  uint8_t depth[64] = {};
  uint64_t mask[64] = {};
};

// Builds a Tree from a host parent array; false unless parent[0] = -1, 0 <= parent[i] < i, n <= 64
// and every depth <= max_depth_allowed.
bool make_tree(const int32_t* parent, int n, int max_depth_allowed, Tree* t) {
  if (!parent || n < 1 || n > 64 || parent[0] != -1) return false;
  t->n = n;
  t->max_depth = 0;
  t->parent[0] = -1;
  t->depth[0] = 0;
  t->mask[0] = 1ull;
  for (int i = 1; i < n; ++i) {
    const int p = parent[i];
    if (p < 0 || p >= i) return false;
    t->parent[i] = (int8_t)p;
    t->depth[i] = (uint8_t)(t->depth[p] + 1);
    t->mask[i] = t->mask[p] | (1ull << i);
    t->max_depth = std::max<int>(t->max_depth, t->depth[i]);
  }
  return t->max_depth <= max_depth_allowed;
}

int attention(specdec_ctx* x, int layer, int B, int R, int key_off, int cls, hipStream_t st,
              int vis = VIS_CAUSAL, const Tree* tree = nullptr) {
  const specdec_config& c = x->cfg;
  AttnArgs a;
  const size_t per_layer = (size_t)c.max_batch * c.n_kv_heads * c.max_ctx * c.head_dim;
  a.q = x->ws + x->lay.q;
  a.kcache = (const char*)x->kv_k + per_layer * layer * x->dm.esz;
  a.vcache = (const char*)x->kv_v + per_layer * layer * x->dm.esz;
  a.len = x->len;
  a.out = x->ws + x->lay.o;
  a.out_qx = B * R <= 4;  // the O projection's operand, in the quad layout for up to 4 rows
  a.part = at<float>(x, x->lay.att_part);
  a.err = at<int>(x, x->lay.err);
  a.B = B;
  a.R = R;
  a.key_off = key_off;
  a.hq = c.n_q_heads;
  a.hkv = c.n_kv_heads;
  a.hd = c.head_dim;
  a.max_ctx = c.max_ctx;
  a.cache_b_stride = c.n_kv_heads * c.max_ctx * c.head_dim;
  a.chunk = x->dm.chunk;
  a.n_chunks = x->dm.n_chunks;
  int hi = 0;  // chunks that can hold a visible key, from the host-side bound on len
  for (int b = 0; b < B; ++b) hi = std::max(hi, x->len_hi[b]);
  a.n_launch = std::min(x->dm.n_chunks, std::max(1, cdiv(std::min(attn_key_end(vis, hi, R, key_off),
                                                                  c.max_ctx),
                                                         x->dm.chunk)));
  a.scale = 1.0f / std::sqrt((float)c.head_dim);
  a.vis = vis;
  a.q_split = attention_q_split(a.n_launch, a.hkv, B, R, c.n_q_heads / c.n_kv_heads);
  if (tree) a.tree_mask = at<uint64_t>(x, x->lay.tree_mask);
  ProfScope ps(x, cls, st);
  HIP_TRY(launch_attention(dt_of(x), a, st));
  return SPECDEC_OK;
}

int static_workspace(void** out);
int create_on(const specdec_config* cfg, const specdec_weights* w, void* kv_k, void* kv_v,
              int32_t* len, float* hid, void* workspace, size_t workspace_bytes, void* stream,
              specdec_ctx** out);

}  // namespace

extern "C" {

size_t specdec_workspace_bytes(const specdec_config* cfg) {
  if (!valid_config(cfg)) return 0;
  return make_layout(cfg, make_dims(cfg)).total;
}

size_t specdec_kv_elems(const specdec_config* c) {
  if (!valid_config(c)) return 0;
  return (size_t)c->n_layers * c->max_batch * c->n_kv_heads * c->max_ctx * c->head_dim;
}

int specdec_create(const specdec_config* cfg, const specdec_weights* w, void* kv_k, void* kv_v,
                   int32_t* len, float* hid, void* workspace, size_t workspace_bytes,
                   void* stream, specdec_ctx** out) {
  if (!out) return SPECDEC_E_INVAL;
  *out = nullptr;
  if (!valid_config(cfg) || !w || !kv_k || !kv_v || !len || !hid || !workspace)
    return SPECDEC_E_INVAL;
  return create_on(cfg, w, kv_k, kv_v, len, hid, workspace, workspace_bytes, stream, out);
}

int specdec_create_static(const specdec_config* cfg, const specdec_weights* w, void* kv_k,
                          void* kv_v, int32_t* len, float* hid, void* stream, specdec_ctx** out) {
  if (!out) return SPECDEC_E_INVAL;
  *out = nullptr;
  if (!valid_config(cfg) || !w || !kv_k || !kv_v || !len || !hid) return SPECDEC_E_INVAL;
  const size_t need = specdec_workspace_bytes(cfg);
  if (need > SPECDEC_STATIC_WORKSPACE_BYTES) return SPECDEC_E_CAPACITY;
  void* ws = nullptr;
  const int rc = static_workspace(&ws);
  if (rc != SPECDEC_OK) return rc;
  return create_on(cfg, w, kv_k, kv_v, len, hid, ws, SPECDEC_STATIC_WORKSPACE_BYTES, stream, out);
}

}  // extern "C"

namespace {

// Address of this GPU's copy of `scratch`, looked up once per device with that device current.
int static_workspace(void** out) {
  static std::mutex mu;
  static void* addr[256] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return SPECDEC_E_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPECDEC_E_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return SPECDEC_OK;
}

int create_on(const specdec_config* cfg, const specdec_weights* w, void* kv_k, void* kv_v,
              int32_t* len, float* hid, void* workspace, size_t workspace_bytes, void* stream,
              specdec_ctx** out) {
  if (!attention_supported(cfg->head_dim)) return SPECDEC_E_UNSUPPORTED;
  if (((uintptr_t)workspace) % ALIGN) return SPECDEC_E_INVAL;
  if (!w->embed || !w->final_norm || !w->layers || !w->table || !w->centroids || !w->row_vocab ||
      !w->vocab_row || !w->norm_h || !w->norm_e || !w->w_in || !w->d_layers || !w->norm_f ||
      !w->w_back)
    return SPECDEC_E_INVAL;
  const int slots_used = cfg->n_experts > 0 ? SPECDEC_N_LAYER_TENSORS : SPECDEC_LW_ROUTER;
  for (int l = 0; l < cfg->n_layers; ++l)
    for (int i = 0; i < slots_used; ++i)
      if (!w->layers[(size_t)l * SPECDEC_N_LAYER_TENSORS + i]) return SPECDEC_E_INVAL;
  for (int i = 0; i < cfg->d_layers * SPECDEC_N_DRAFT_TENSORS; ++i)
    if (!w->d_layers[i]) return SPECDEC_E_INVAL;
  if (workspace_bytes < specdec_workspace_bytes(cfg)) return SPECDEC_E_INVAL;

  specdec_ctx* x = new (std::nothrow) specdec_ctx();
  if (!x) return SPECDEC_E_INVAL;
  x->cfg = *cfg;
  if (x->cfg.kv_src_layer < 0) x->cfg.kv_src_layer = cfg->n_layers - 1;
  x->dm = make_dims(cfg);
  x->lay = make_layout(cfg, x->dm);
  x->ws = reinterpret_cast<char*>(workspace);
  x->kv_k = kv_k;
  x->kv_v = kv_v;
  x->len = len;
  x->hid = hid;
  x->w = *w;
  x->lw.assign(w->layers, w->layers + (size_t)cfg->n_layers * SPECDEC_N_LAYER_TENSORS);
  x->dw.assign(w->d_layers, w->d_layers + (size_t)cfg->d_layers * SPECDEC_N_DRAFT_TENSORS);
  x->w.layers = nullptr;
  x->w.d_layers = nullptr;
  build_gemms(x);
  x->len_hi.assign(cfg->max_batch, 0);
  if (launch_fill_i32(at<int>(x, x->lay.err), 0, 16, reinterpret_cast<hipStream_t>(stream)) !=
          hipSuccess ||
      launch_rope_table(at<float2>(x, x->lay.rope), cfg->head_dim, cfg->max_ctx, cfg->rope_theta,
                        reinterpret_cast<hipStream_t>(stream)) != hipSuccess) {
    delete x;
    return SPECDEC_E_HIP;
  }
  *out = x;
  return SPECDEC_OK;
}

}  // namespace

extern "C" {

int specdec_destroy(specdec_ctx* x) {
  if (!x) return SPECDEC_E_INVAL;
  for (auto e : x->prof_ev) (void)hipEventDestroy(e);
  delete x;
  return SPECDEC_OK;
}

}  // extern "C"

namespace {

// The target's forward over R rows per sequence (validated by the caller): linear rows (row i at
// position len + i, seeing keys up to its own slot) or the nodes of a token tree.
int verify_impl(specdec_ctx* x, int B, int R, const int32_t* tokens, float* logits, int32_t* argmax,
                const Tree* tree, hipStream_t st) {
  const specdec_config& c = x->cfg;
  const int M = B * R;
  if (tree)
    HIP_TRY(launch_tree_desc(tree->n, tree->mask, tree->depth, at<uint64_t>(x, x->lay.tree_mask),
                             at<uint8_t>(x, x->lay.tree_depth), st));
  const int d = c.d_model, qd = c.n_q_heads * c.head_dim;
  float* X = at<float>(x, x->lay.x);
  void* XW = x->ws + x->lay.xw;
  float* ssq = at<float>(x, x->lay.ssq);
  int* err = at<int>(x, x->lay.err);
  auto lw = [&](int l, int slot) { return (const float*)x->lw[(size_t)l * SPECDEC_N_LAYER_TENSORS + slot]; };
  HIP_TRY(launch_embed(dt_of(x), x->w.embed, x->g_head.nkb, d, tokens, M, X, ssq, XW, M <= 4,
                       lw(0, SPECDEC_LW_ATTN_NORM), c.vocab, err, st,
                       c.weight_format == SPECDEC_WF_Q4));
  const size_t per_layer = (size_t)c.max_batch * c.n_kv_heads * c.max_ctx * c.head_dim;
  int rc;
  for (int l = 0; l < c.n_layers; ++l) {
    {  // fused q/k/v projection + RoPE + KV append (tentative: len is not moved)
      GemmArgs a = base_args(x, x->g_qkv[l], M);
      norm_input(a, XW, d, ssq, d);
      a.qout = x->ws + x->lay.q;
      a.kcache = (char*)x->kv_k + per_layer * l * x->dm.esz;
      a.vcache = (char*)x->kv_v + per_layer * l * x->dm.esz;
      a.len = x->len;
      a.rows_per_seq = R;
      a.pos_off = 0;
      a.hq = c.n_q_heads;
      a.hkv = c.n_kv_heads;
      a.hd = c.head_dim;
      a.max_ctx = c.max_ctx;
      a.cache_b_stride = c.n_kv_heads * c.max_ctx * c.head_dim;
      a.theta = c.rope_theta;
      a.rope_cs = at<float2>(x, x->lay.rope);
      if (tree) {
        a.pos_mode = POS_TREE;
        a.tree_depth = at<uint8_t>(x, x->lay.tree_depth);
      }
      if ((rc = run(x, 2, EPI_ROPE, a, st))) return rc;
    }
    if ((rc = attention(x, l, B, R, 1, 4, st, tree ? VIS_TREE : VIS_CAUSAL, tree))) return rc;
    {  // output projection + residual; leaves x * ffn_norm for the FFN
      GemmArgs a = base_args(x, x->g_o[l], M);
      a.X = x->ws + x->lay.o;
      a.ldx = qd;
      resid_output(a, X, d, 1, ssq, XW, lw(l, SPECDEC_LW_FFN_NORM));
      if ((rc = run(x, 3, EPI_STORE, a, st))) return rc;
    }
    if (c.n_experts > 0 && (rc = routed_experts(x, l, M, st))) return rc;
    const int Fw = ffn_width(&c);
    {  // gate/up projection + SiLU-gated product (the shared FFN of an MoE layer)
      GemmArgs a = base_args(x, x->g_gu[l], M);
      wide_units(a, x->g_gu[l], M);
      norm_input(a, XW, d, ssq, d);
      a.hout = x->ws + x->lay.h;
      a.ldh = Fw;
      if ((rc = run(x, 0, EPI_SILU, a, st))) return rc;
    }
    {  // down projection + residual (+ the routed experts' weighted outputs, ascending expert
       // id); leaves x * (next attention norm | final norm)
      GemmArgs a = base_args(x, x->g_down[l], M);
      a.X = x->ws + x->lay.h;
      a.ldx = Fw;
      const float* wn = l + 1 < c.n_layers ? lw(l + 1, SPECDEC_LW_ATTN_NORM) : x->w.final_norm;
      resid_output(a, X, d, 1, ssq, XW, wn);
      if (c.n_experts > 0) {
        a.addend = at<float>(x, x->lay.e_y);
        a.add_n = c.top_k;
      }
      if ((rc = run(x, 1, EPI_STORE, a, st))) return rc;
    }
  }
  {  // final norm + tied LM head with per-unit argmax partials
    GemmArgs a = base_args(x, x->g_head, M);
    norm_input(a, XW, d, ssq, d);
    a.amax_val = at<float>(x, x->lay.amax_v);
    a.amax_idx = at<int>(x, x->lay.amax_i);
    a.ld_amax = x->dm.parts;
    a.logits = logits;
    a.ld_logits = c.vocab;
    if ((rc = run(x, 5, EPI_ARGMAX, a, st))) return rc;
  }
  if (argmax) {
    HIP_TRY(launch_accept(at<float>(x, x->lay.amax_v), at<int>(x, x->lay.amax_i), x->dm.parts,
                          x->dm.parts, B, R, nullptr, nullptr, nullptr, nullptr, 0, x->len,
                          x->hid, X, d, argmax, err, st));
  }
  x->last_B = B;
  x->last_R = R;
  x->last_tree_n = tree ? tree->n : 0;
  if (tree)
    for (int i = 0; i < tree->n; ++i) x->last_parent[i] = tree->parent[i];
  return SPECDEC_OK;
}

// Ways the reduction of a prompt GEMM is split.  A projection whose 256 x 256 blocks leave most
// CUs idle takes up to MM_SPLIT_WGS workgroups, each at least 8 k-blocks of the reduction, with
// the fp32 partials (4 bytes per split and output) at most the weight bytes.  Measured on MI355X
// at the 31B shapes, 512 rows: o + down 500 -> 231 us per layer including the summing launches;
// q/k/v 158 -> 82 us (its summing launch stores the rotary outputs through LDS).
int mm_split(const Gemm& g, int M, int epi) {
  const int blocks = cdiv(g.n_tiles, 16) * cdiv(M, 256);
  if (blocks >= MM_SPLIT_WGS / 4) return 1;
  const int kn = std::min({MM_SPLIT_WGS / blocks, g.nkb / 8, 16 * g.nkb / M});
  return kn >= 2 ? kn : 1;
}

// The GEMM arguments of a prompt-chunk launch (launch_mm): the weights, the row count and the
// split of the reduction (partials in the attention partials' buffer, free outside attention).
GemmArgs mm_args(specdec_ctx* x, const Gemm& g, int M, int epi) {
  GemmArgs a;
  a.W = g.W;
  a.nkb = g.nkb;
  a.n_tiles = g.n_tiles;
  a.M = M;
  a.err = at<int>(x, x->lay.err);
  a.eps = x->cfg.rms_eps;
  a.wq4 = x->cfg.weight_format == SPECDEC_WF_Q4;
  a.kpart_n = mm_split(g, M, epi);
  if (a.kpart_n > 1) a.kpart = at<float>(x, x->lay.p_part);
  return a;
}

// Prompt chunk of T rows of sequence b through the target (the same layer sequence as a verify),
// on the compute-bound GEMM and the attention split over key chunks and query blocks, then the
// commit of all T rows.
int prefill_impl(specdec_ctx* x, int b, int T, const int32_t* tokens, float* logits,
                 int32_t* argmax, hipStream_t st) {
  const specdec_config& c = x->cfg;
  const int d = c.d_model, qd = c.n_q_heads * c.head_dim, Fw = c.ffn_dim;
  float* X = at<float>(x, x->lay.p_x);
  void* XW = x->ws + x->lay.p_xw;
  float* ssq = at<float>(x, x->lay.p_ssq);
  int* err = at<int>(x, x->lay.err);
  int* len = x->len + b;
  auto lw = [&](int l, int slot) { return (const float*)x->lw[(size_t)l * SPECDEC_N_LAYER_TENSORS + slot]; };
  HIP_TRY(launch_embed(DT_BF16, x->w.embed, x->g_head.nkb, d, tokens, T, X, ssq, XW, 0,
                       lw(0, SPECDEC_LW_ATTN_NORM), c.vocab, err, st,
                       c.weight_format == SPECDEC_WF_Q4));
  const size_t per_layer = (size_t)c.max_batch * c.n_kv_heads * c.max_ctx * c.head_dim;
  const size_t seq = (size_t)b * c.n_kv_heads * c.max_ctx * c.head_dim;  // sequence b's cache
  for (int l = 0; l < c.n_layers; ++l) {
    void* kc = (char*)x->kv_k + (per_layer * l + seq) * 2;
    void* vc = (char*)x->kv_v + (per_layer * l + seq) * 2;
    {  // q/k/v projection + RoPE at positions len + row + K/V append
      GemmArgs a = mm_args(x, x->g_qkv[l], T, EPI_ROPE);
      norm_input(a, XW, d, ssq, d);
      a.qout = x->ws + x->lay.p_q;
      a.kcache = kc;
      a.vcache = vc;
      a.len = len;
      a.hq = c.n_q_heads;
      a.hkv = c.n_kv_heads;
      a.hd = c.head_dim;
      a.max_ctx = c.max_ctx;
      a.rope_cs = at<float2>(x, x->lay.rope);
      HIP_TRY(launch_mm(EPI_ROPE, a, st));
    }
    {  // causal attention of the T rows over the committed prefix and the chunk
      AttnArgs a;
      a.q = x->ws + x->lay.p_q;
      a.kcache = kc;
      a.vcache = vc;
      a.len = len;
      a.out = x->ws + x->lay.p_o;
      a.out_qx = 0;
      a.err = err;
      a.B = 1;
      a.R = T;
      a.key_off = 1;
      a.hq = c.n_q_heads;
      a.hkv = c.n_kv_heads;
      a.hd = c.head_dim;
      a.max_ctx = c.max_ctx;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      a.vis = VIS_CAUSAL;
      // split the keys into ranges (merged by the combine) when the query-vector blocks alone
      // leave the CUs with few waves: about PROMPT_ATTN_WGS workgroups in all; fewer than
      // PROMPT_SPLIT_KEYS keys are walked whole
      const int G = c.n_q_heads / c.n_kv_heads;
      const int blocks = cdiv(T * G, attention_prompt_block(T, c.n_q_heads, c.n_kv_heads)) * c.n_kv_heads;
      const int kend = x->len_hi[b] + T;  // bound on the keys any row sees
      const int ranges = kend < PROMPT_SPLIT_KEYS
                             ? 1 : std::max(1, std::min(PROMPT_MAX_RANGES, PROMPT_ATTN_WGS / blocks));
      a.chunk = cdiv(cdiv(kend, ranges), 64) * 64;
      a.n_chunks = a.n_launch = cdiv(kend, a.chunk);
      if (a.n_chunks > 1) a.part = at<float>(x, x->lay.p_part);
      HIP_TRY(launch_attention_prompt(a, st));
    }
    {  // output projection + residual; leaves x * ffn_norm
      GemmArgs a = mm_args(x, x->g_o[l], T, EPI_STORE);
      a.X = x->ws + x->lay.p_o;
      a.ldx = qd;
      resid_output(a, X, d, 1, ssq, XW, lw(l, SPECDEC_LW_FFN_NORM));
      HIP_TRY(launch_mm(EPI_STORE, a, st));
    }
    {  // gate/up + SiLU product
      GemmArgs a = mm_args(x, x->g_gu[l], T, EPI_SILU);
      norm_input(a, XW, d, ssq, d);
      a.hout = x->ws + x->lay.p_h;
      a.ldh = Fw;
      HIP_TRY(launch_mm(EPI_SILU, a, st));
    }
    {  // down projection + residual; leaves x * (next attention norm | final norm)
      GemmArgs a = mm_args(x, x->g_down[l], T, EPI_STORE);
      a.X = x->ws + x->lay.p_h;
      a.ldx = Fw;
      const float* wn = l + 1 < c.n_layers ? lw(l + 1, SPECDEC_LW_ATTN_NORM) : x->w.final_norm;
      resid_output(a, X, d, 1, ssq, XW, wn);
      HIP_TRY(launch_mm(EPI_STORE, a, st));
    }
  }
  {  // final norm + tied LM head: per-unit argmax partials (+ optional logits)
    GemmArgs a = mm_args(x, x->g_head, T, EPI_ARGMAX);
    norm_input(a, XW, d, ssq, d);
    a.amax_val = at<float>(x, x->lay.p_amax_v);
    a.amax_idx = at<int>(x, x->lay.p_amax_i);
    a.ld_amax = x->dm.parts;
    a.logits = logits;
    a.ld_logits = c.vocab;
    HIP_TRY(launch_mm(EPI_ARGMAX, a, st));
  }
  if (argmax)
    HIP_TRY(launch_rows_argmax(at<float>(x, x->lay.p_amax_v), at<int>(x, x->lay.p_amax_i),
                               x->dm.parts, x->dm.parts, T, argmax, st));
  HIP_TRY(launch_commit_rows(len, x->hid + (size_t)b * d, X + (size_t)(T - 1) * d, d, T, st));
  x->len_hi[b] += T;
  x->last_B = 0;  // a verify's rows can no longer be accepted or committed
  x->last_R = 0;
  x->last_tree_n = 0;
  return SPECDEC_OK;
}

}  // namespace

extern "C" {

int specdec_prefill(specdec_ctx* x, int32_t b, int32_t T, const int32_t* tokens, float* logits,
                    int32_t* argmax, void* stream) {
  if (!x || !tokens) return SPECDEC_E_INVAL;
  const specdec_config& c = x->cfg;
  if (c.max_prefill < 1) return SPECDEC_E_UNSUPPORTED;
  if (b < 0 || b >= c.max_batch || T < 1 || T > c.max_prefill) return SPECDEC_E_INVAL;
  if (x->len_hi[b] + T > c.max_ctx) return SPECDEC_E_CAPACITY;
  return prefill_impl(x, b, T, tokens, logits, argmax, reinterpret_cast<hipStream_t>(stream));
}

int specdec_verify(specdec_ctx* x, int32_t B, int32_t R, const int32_t* tokens, float* logits,
                   int32_t* argmax, void* stream) {
  if (!x || !tokens) return SPECDEC_E_INVAL;
  const specdec_config& c = x->cfg;
  if (B < 1 || B > c.max_batch || R < 1 || R > c.max_rows) return SPECDEC_E_INVAL;
  for (int b = 0; b < B; ++b)
    if (x->len_hi[b] + R > c.max_ctx) return SPECDEC_E_CAPACITY;
  return verify_impl(x, B, R, tokens, logits, argmax, nullptr, reinterpret_cast<hipStream_t>(stream));
}

int specdec_verify_tree(specdec_ctx* x, int32_t B, int32_t n_nodes, const int32_t* parent,
                        const int32_t* tokens, float* logits, int32_t* argmax, void* stream) {
  if (!x || !tokens || !parent) return SPECDEC_E_INVAL;
  const specdec_config& c = x->cfg;
  if (B < 1 || B > c.max_batch || n_nodes < 1 || n_nodes > c.max_rows) return SPECDEC_E_INVAL;
  Tree t;
  if (!make_tree(parent, n_nodes, SPECDEC_TREE_MAX_DEPTH, &t)) return SPECDEC_E_INVAL;
  for (int b = 0; b < B; ++b)
    if (x->len_hi[b] + n_nodes > c.max_ctx) return SPECDEC_E_CAPACITY;
  return verify_impl(x, B, n_nodes, tokens, logits, argmax, &t, reinterpret_cast<hipStream_t>(stream));
}

int specdec_accept_tree(specdec_ctx* x, int32_t B, int32_t n_nodes, const int32_t* parent,
                        const int32_t* tokens, int32_t* out_tokens, int32_t out_ld,
                        int32_t* n_emit, int32_t* next_tok, uint32_t flags, void* stream) {
  if (!x || !tokens || !parent || !out_tokens) return SPECDEC_E_INVAL;
  if (B != x->last_B || n_nodes != x->last_tree_n || n_nodes != x->last_R) return SPECDEC_E_INVAL;
  Tree t;
  if (!make_tree(parent, n_nodes, SPECDEC_TREE_MAX_DEPTH, &t)) return SPECDEC_E_INVAL;
  for (int i = 0; i < n_nodes; ++i)
    if (t.parent[i] != x->last_parent[i]) return SPECDEC_E_INVAL;  // not the verified tree
  if (out_ld < t.max_depth + 1) return SPECDEC_E_INVAL;
  const bool commit = (flags & SPECDEC_ACCEPT_COMMIT) != 0;
  const specdec_config& c = x->cfg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int* path = at<int>(x, x->lay.path);
  HIP_TRY(launch_tree_accept(at<float>(x, x->lay.amax_v), at<int>(x, x->lay.amax_i), x->dm.parts,
                             x->dm.parts, B, n_nodes, t.parent, tokens, out_tokens, out_ld, n_emit,
                             next_tok, commit ? 1 : 0, x->len, x->hid, at<float>(x, x->lay.x),
                             c.d_model, path, at<int>(x, x->lay.err), st));
  if (commit) {
    // the accepted path's cache entries move to the slots after the committed prefix
    HIP_TRY(launch_kv_compact(dt_of(x), x->kv_k, x->kv_v, path, c.n_layers, B, c.max_batch,
                              c.n_kv_heads, c.head_dim, c.max_ctx, st));
    for (int b = 0; b < B; ++b) x->len_hi[b] += t.max_depth + 1;
  }
  return SPECDEC_OK;
}

int specdec_accept(specdec_ctx* x, int32_t B, int32_t K, const int32_t* tokens,
                   int32_t* out_tokens, int32_t* n_emit, int32_t* next_tok, uint32_t flags,
                   void* stream) {
  if (!x || !tokens) return SPECDEC_E_INVAL;
  if (B != x->last_B || K + 1 != x->last_R || K < 0 || x->last_tree_n) return SPECDEC_E_INVAL;
  const bool commit = (flags & SPECDEC_ACCEPT_COMMIT) != 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_accept(at<float>(x, x->lay.amax_v), at<int>(x, x->lay.amax_i), x->dm.parts,
                        x->dm.parts, B, K + 1, tokens, out_tokens, n_emit, next_tok,
                        commit ? 1 : 0, x->len, x->hid, at<float>(x, x->lay.x), x->cfg.d_model,
                        nullptr, at<int>(x, x->lay.err), st));
  if (commit)
    for (int b = 0; b < B; ++b) x->len_hi[b] += K + 1;
  return SPECDEC_OK;
}

int specdec_kv_commit(specdec_ctx* x, int32_t B, const int32_t* n_commit, void* stream) {
  if (!x || !n_commit || B != x->last_B || B < 1 || x->last_tree_n) return SPECDEC_E_INVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_commit(n_commit, B, x->last_R, x->len, x->hid, at<float>(x, x->lay.x),
                        x->cfg.d_model, at<int>(x, x->lay.err), st));
  for (int b = 0; b < B; ++b) x->len_hi[b] += x->last_R;
  return SPECDEC_OK;
}

int specdec_draft(specdec_ctx* x, int32_t B, int32_t K, int32_t head_mode, int32_t k_c,
                  const int32_t* cur_tok, int32_t* drafts, const int32_t* inject,
                  int64_t inj_stride, int32_t* verify_tokens, void* stream) {
  return specdec_draft_traced(x, B, K, head_mode, k_c, cur_tok, drafts, inject, inj_stride,
                              verify_tokens, nullptr, stream);
}

}  // extern "C"

namespace {

// One drafter sub-step over `rows` rows, rps rows per sequence (a tree draft's branches; 1 for a
// linear draft) sharing their sequence's cache and query position len + pos_off.  Row r reads
// hidden input h[r / h_div] and token tok[r].  Leaves x * n_f and its sums of squares for the head
// and the next hidden input W_back s in hnext[r].
int drafter_body(specdec_ctx* x, int rows, int rps, const float* h, int h_div, const int* tok,
                 int pos_off, hipStream_t st) {
  const specdec_config& c = x->cfg;
  const int d = c.d_model, Dd = c.d_dim, qd = c.n_q_heads * c.head_dim;
  float* xd = at<float>(x, x->lay.xd);
  void* xdw = x->ws + x->lay.xdw;
  float* sd = at<float>(x, x->lay.ssq_d);
  int* err = at<int>(x, x->lay.err);
  auto dw = [&](int l, int slot) { return (const float*)x->dw[(size_t)l * SPECDEC_N_DRAFT_TENSORS + slot]; };
  int rc;
  HIP_TRY(launch_draft_input(dt_of(x), h, tok, x->w.table, x->g_table.nkb, x->w.vocab_row, c.vocab,
                             x->w.norm_h, x->w.norm_e, d, Dd, c.rms_eps, x->ws + x->lay.u,
                             rows <= 4, rows, err, st, h_div, c.weight_format == SPECDEC_WF_Q4));
  {  // input projection of [rms(h); rms(e)]; leaves x * n1 of the first drafter layer
    GemmArgs a = base_args(x, x->g_in, rows);
    a.X = x->ws + x->lay.u;
    a.ldx = d + Dd;
    resid_output(a, xd, Dd, 0, sd, xdw, dw(0, SPECDEC_DW_N1));
    if ((rc = run(x, -1, EPI_STORE, a, st))) return rc;
  }
  for (int l = 0; l < c.d_layers; ++l) {
    {  // q projection + RoPE at len + pos_off (every row of a sequence at the same position)
      GemmArgs a = base_args(x, x->g_dq[l], rows);
      norm_input(a, xdw, Dd, sd, Dd);
      a.qout = x->ws + x->lay.q;
      a.len = x->len;
      a.rows_per_seq = rps;
      a.pos_off = pos_off;
      a.pos_mode = POS_FLAT;
      a.hq = c.n_q_heads;
      a.hkv = 0;
      a.hd = c.head_dim;
      a.max_ctx = c.max_ctx;
      a.theta = c.rope_theta;
      a.rope_cs = at<float2>(x, x->lay.rope);
      if ((rc = run(x, -1, EPI_ROPE, a, st))) return rc;
    }
    // cross-attention into the target's cache, keys [0, len) for every row
    if ((rc = attention(x, c.kv_src_layer, rows / rps, rps, 0, -1, st, VIS_FLAT))) return rc;
    {  // o projection + residual; leaves x * n2
      GemmArgs a = base_args(x, x->g_do[l], rows);
      a.X = x->ws + x->lay.o;
      a.ldx = qd;
      resid_output(a, xd, Dd, 1, sd, xdw, dw(l, SPECDEC_DW_N2));
      if ((rc = run(x, -1, EPI_STORE, a, st))) return rc;
    }
    {
      GemmArgs a = base_args(x, x->g_dgu[l], rows);
      norm_input(a, xdw, Dd, sd, Dd);
      a.hout = x->ws + x->lay.dh;
      a.ldh = c.d_ffn;
      if ((rc = run(x, -1, EPI_SILU, a, st))) return rc;
    }
    {  // down projection + residual; leaves x * (next n1 | n_f)
      GemmArgs a = base_args(x, x->g_ddown[l], rows);
      a.X = x->ws + x->lay.dh;
      a.ldx = c.d_ffn;
      const float* wn = l + 1 < c.d_layers ? dw(l + 1, SPECDEC_DW_N1) : x->w.norm_f;
      resid_output(a, xd, Dd, 1, sd, xdw, wn);
      if ((rc = run(x, -1, EPI_STORE, a, st))) return rc;
    }
  }
  {  // next hidden input: W_back . (rms(x) * n_f)
    GemmArgs a = base_args(x, x->g_back, rows);
    norm_input(a, xdw, Dd, sd, Dd);
    a.out = at<float>(x, x->lay.hnext);
    a.ldo = d;
    if ((rc = run(x, -1, EPI_STORE, a, st))) return rc;
  }
  return SPECDEC_OK;
}

// Where a head's argmax partials sit: row r's parts are amax[r * ld + r * seq_off + p], p < parts.
struct HeadParts {
  int parts, seq_off, ld;
};

// The drafter's output layer over `rows` rows: SPECDEC_HEAD_FULL scores every table row,
// SPECDEC_HEAD_CLUSTERED scores the centroids, selects k_c clusters per row and scores their
// members.  Optional copies: the scores by table row (scores, row stride ld_scores) and the
// centroid scores (zcopy, row stride ld_z).
int drafter_head(specdec_ctx* x, int rows, int head_mode, int k_c, float* scores, int ld_scores,
                 float* zcopy, int ld_z, HeadParts* hp, hipStream_t st) {
  const specdec_config& c = x->cfg;
  const int dt = dt_of(x), Dd = c.d_dim;
  const int S = c.vocab / c.n_centroids;  // tokens per cluster
  const int tpc = S / 16, upc = S / 64;   // tiles / argmax units per cluster
  void* xdw = x->ws + x->lay.xdw;
  float* sd = at<float>(x, x->lay.ssq_d);
  ProfScope ps(x, 6, st);
  if (head_mode == SPECDEC_HEAD_FULL) {
    GemmArgs a = base_args(x, x->g_table, rows);
    norm_input(a, xdw, Dd, sd, Dd);
    a.amax_val = at<float>(x, x->lay.d_amax_v);
    a.amax_idx = at<int>(x, x->lay.d_amax_i);
    a.ld_amax = x->dm.parts;
    a.idx_map = x->w.row_vocab;
    a.logits = scores;
    a.ld_logits = ld_scores;
    HIP_TRY(launch_gemm(dt, mt_for(rows), 4, EPI_ARGMAX, a, st));
    *hp = {x->dm.parts, 0, x->dm.parts};
    return SPECDEC_OK;
  }
  GemmArgs zc = base_args(x, x->g_cent, rows);
  norm_input(zc, xdw, Dd, sd, Dd);
  zc.out = at<float>(x, x->lay.z);
  zc.ldo = c.n_centroids;
  HIP_TRY(launch_gemm(dt, mt_for(rows), 1, EPI_STORE, zc, st));
  if (zcopy)
    HIP_TRY(launch_copy_rows(zcopy, ld_z, zc.out, c.n_centroids, rows, c.n_centroids, st));
  HIP_TRY(launch_cluster_select(at<float>(x, x->lay.z), c.n_centroids, k_c, rows, tpc, upc,
                                at<int>(x, x->lay.utile), at<int>(x, x->lay.urow),
                                at<int>(x, x->lay.err), st));
  GemmArgs a = base_args(x, x->g_clu, rows);
  a.n_units = rows * k_c * upc;
  a.unit_tile = at<int>(x, x->lay.utile);
  a.unit_row = at<int>(x, x->lay.urow);
  norm_input(a, xdw, Dd, sd, Dd);
  a.amax_val = at<float>(x, x->lay.d_amax_v);
  a.amax_idx = at<int>(x, x->lay.d_amax_i);
  a.idx_map = x->w.row_vocab;
  a.logits = scores;
  a.ld_logits = ld_scores;
  HIP_TRY(launch_gemm(dt, mt_for(rows), 4, EPI_ARGMAX, a, st));
  *hp = {k_c * upc, k_c * upc, 0};  // listed units are stored by unit index
  return SPECDEC_OK;
}

int check_head(const specdec_config& c, int head_mode, int k_c) {
  if (head_mode != SPECDEC_HEAD_CLUSTERED && head_mode != SPECDEC_HEAD_FULL) return SPECDEC_E_INVAL;
  if (head_mode == SPECDEC_HEAD_CLUSTERED && (k_c < 1 || k_c > c.n_centroids)) return SPECDEC_E_INVAL;
  return SPECDEC_OK;
}

}  // namespace

extern "C" {

int specdec_draft_traced(specdec_ctx* x, int32_t B, int32_t K, int32_t head_mode, int32_t k_c,
                         const int32_t* cur_tok, int32_t* drafts, const int32_t* inject,
                         int64_t inj_stride, int32_t* verify_tokens,
                         const specdec_draft_trace* trace, void* stream) {
  if (!x || !cur_tok || !drafts) return SPECDEC_E_INVAL;
  const specdec_config& c = x->cfg;
  if (B < 1 || B > c.max_batch || K < 1 || K > c.max_draft) return SPECDEC_E_INVAL;
  if (check_head(c, head_mode, k_c)) return SPECDEC_E_INVAL;
  if (inject && (inj_stride < 1 || inj_stride > 0x7fffffff)) return SPECDEC_E_INVAL;
  // sub-step j queries at position len + j - 1: the last one, len + K - 1, must be a cache slot
  for (int b = 0; b < B; ++b)
    if (x->len_hi[b] + K > c.max_ctx) return SPECDEC_E_CAPACITY;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int d = c.d_model, Dd = c.d_dim;
  float* hnext = at<float>(x, x->lay.hnext);
  int* dtok = at<int>(x, x->lay.dtok);
  int rc;
  for (int j = 1; j <= K; ++j) {
    const float* h = (j == 1) ? x->hid : hnext;
    const int* tok = (j == 1) ? cur_tok : dtok;
    if ((rc = drafter_body(x, B, 1, h, 1, tok, j - 1, st))) return rc;
    if (trace && trace->state)
      HIP_TRY(launch_trace_state(at<float>(x, x->lay.xd), at<float>(x, x->lay.ssq_d), B, Dd,
                                 x->w.norm_f, c.rms_eps, trace->state + (size_t)(j - 1) * Dd,
                                 K * Dd, st));
    if (trace && trace->hidden)
      HIP_TRY(launch_copy_rows(trace->hidden + (size_t)(j - 1) * d, K * d, hnext, d, B, d, st));
    // the head's scores of sub-step j land at trace row b*K + j - 1, by table row
    float* tscores = trace && trace->table_scores ? trace->table_scores + (size_t)(j - 1) * c.vocab : nullptr;
    float* zcopy = trace && trace->centroid_scores
                       ? trace->centroid_scores + (size_t)(j - 1) * c.n_centroids : nullptr;
    HeadParts hp;
    if ((rc = drafter_head(x, B, head_mode, k_c, tscores, K * c.vocab, zcopy, K * c.n_centroids, &hp, st)))
      return rc;
    HIP_TRY(launch_draft_finalize(at<float>(x, x->lay.d_amax_v), at<int>(x, x->lay.d_amax_i), hp.ld,
                                  hp.parts, hp.seq_off, B, K, j, x->len, inject, (int)inj_stride,
                                  drafts, dtok, cur_tok, verify_tokens, at<int>(x, x->lay.err), st));
    if (trace && trace->raw_drafts)
      HIP_TRY(launch_copy_rows(trace->raw_drafts + (j - 1), K, dtok, 1, B, 1, st));
  }
  return SPECDEC_OK;
}

int specdec_draft_tree(specdec_ctx* x, int32_t B, int32_t width, int32_t depth, int32_t head_mode,
                       int32_t k_c, const int32_t* cur_tok, int32_t* tree_tokens,
                       const int32_t* inject, int64_t inj_stride, void* stream) {
  if (!x || !cur_tok || !tree_tokens) return SPECDEC_E_INVAL;
  const specdec_config& c = x->cfg;
  const int n_nodes = 1 + width * depth;
  if (B < 1 || B > c.max_batch || width < 1 || width > SPECDEC_TREE_MAX_WIDTH || depth < 1 ||
      depth > SPECDEC_TREE_MAX_DEPTH || n_nodes > c.max_rows || B * width > x->dm.Mx)
    return SPECDEC_E_INVAL;
  if (check_head(c, head_mode, k_c)) return SPECDEC_E_INVAL;
  if (head_mode == SPECDEC_HEAD_CLUSTERED && width > k_c * (c.vocab / c.n_centroids))
    return SPECDEC_E_INVAL;
  if (inject && (inj_stride < 1 || inj_stride > 0x7fffffff)) return SPECDEC_E_INVAL;
  for (int b = 0; b < B; ++b)
    if (x->len_hi[b] + depth > c.max_ctx) return SPECDEC_E_CAPACITY;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* hnext = at<float>(x, x->lay.hnext);
  int* raw = at<int>(x, x->lay.dtok);
  int* err = at<int>(x, x->lay.err);
  int rc;
  // level 1: one row per sequence; the w best tokens of its head start the branches
  if ((rc = drafter_body(x, B, 1, x->hid, 1, cur_tok, 0, st))) return rc;
  HeadParts hp;
  float* scores = at<float>(x, x->lay.tscore);
  if ((rc = drafter_head(x, B, head_mode, k_c, scores, c.vocab, nullptr, 0, &hp, st))) return rc;
  const bool clu = head_mode == SPECDEC_HEAD_CLUSTERED;
  HIP_TRY(launch_tree_top(scores, c.vocab, clu ? at<int>(x, x->lay.utile) : nullptr, hp.parts, 64,
                          x->w.row_vocab, B, width, depth, cur_tok, x->len, inject, (int)inj_stride,
                          tree_tokens, raw, err, st));
  // levels 2..depth: every branch continues from its own token (the level-1 hidden input is
  // shared by a sequence's branches)
  for (int lv = 2; lv <= depth; ++lv) {
    const int rows = B * width;
    if ((rc = drafter_body(x, rows, width, hnext, lv == 2 ? width : 1, raw, lv - 1, st))) return rc;
    if ((rc = drafter_head(x, rows, head_mode, k_c, nullptr, 0, nullptr, 0, &hp, st))) return rc;
    HIP_TRY(launch_tree_finalize(at<float>(x, x->lay.d_amax_v), at<int>(x, x->lay.d_amax_i), hp.ld,
                                 hp.parts, hp.seq_off, rows, width, depth, lv, x->len, inject,
                                 (int)inj_stride, tree_tokens, raw, err, st));
  }
  return SPECDEC_OK;
}

int specdec_pack_matrix(const void* src, void* dst, int32_t n, int32_t kd, int32_t dtype,
                        int32_t kind, int32_t head_dim, int32_t split_rows, void* stream) {
  if (!src || !dst || n < 16 || kd < 32 || n % 16 || kd % 32) return SPECDEC_E_INVAL;
  if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_E_INVAL;
  if (kind < 0 || kind > 2) return SPECDEC_E_INVAL;
  if (kind == SPECDEC_PACK_ROPE && (head_dim < 16 || head_dim % 16 || n % head_dim))
    return SPECDEC_E_INVAL;
  if (kind == SPECDEC_PACK_GATE_UP && (split_rows < 16 || split_rows % 16 || n % (2 * split_rows)))
    return SPECDEC_E_INVAL;
  HIP_TRY(launch_pack(dtype == SPECDEC_BF16 ? DT_BF16 : DT_F32, src, dst, n, kd, kind, head_dim,
                      split_rows, reinterpret_cast<hipStream_t>(stream)));
  return SPECDEC_OK;
}

size_t specdec_q4_bytes(int32_t n, int32_t kd) {
  if (n < 16 || kd < 128 || n % 16 || kd % 128) return 0;
  return q4_bytes((size_t)n, (size_t)kd);
}

int specdec_pack_q4(const uint8_t* codes, const uint16_t* steps, void* dst, int32_t n, int32_t kd,
                    int32_t kind, int32_t head_dim, int32_t split_rows, void* stream) {
  if (!codes || !steps || !dst || n < 16 || kd < 128 || n % 16 || kd % 128) return SPECDEC_E_INVAL;
  if (reinterpret_cast<uintptr_t>(dst) % 256) return SPECDEC_E_INVAL;
  if (kind < 0 || kind > 2) return SPECDEC_E_INVAL;
  if (kind == SPECDEC_PACK_ROPE && (head_dim < 16 || head_dim % 16 || n % head_dim))
    return SPECDEC_E_INVAL;
  if (kind == SPECDEC_PACK_GATE_UP && (split_rows < 16 || split_rows % 16 || n % (2 * split_rows)))
    return SPECDEC_E_INVAL;
  HIP_TRY(launch_pack_q4(codes, steps, dst, n, kd, kind, head_dim, split_rows,
                         reinterpret_cast<hipStream_t>(stream)));
  return SPECDEC_OK;
}

int specdec_set_len_bound(specdec_ctx* x, const int32_t* host_len, int32_t B) {
  if (!x || !host_len || B < 1 || B > x->cfg.max_batch) return SPECDEC_E_INVAL;
  for (int b = 0; b < B; ++b) {
    if (host_len[b] < 0) return SPECDEC_E_INVAL;
    x->len_hi[b] = host_len[b];
  }
  return SPECDEC_OK;
}

int specdec_read_device_error(specdec_ctx* x, int32_t* host_word, int32_t clear, void* stream) {
  if (!x || !host_word) return SPECDEC_E_INVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(hipMemcpyAsync(host_word, at<int>(x, x->lay.err), 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  if (clear) HIP_TRY(launch_fill_i32(at<int>(x, x->lay.err), 0, 1, st));
  return SPECDEC_OK;
}

int specdec_moe_usage_start(specdec_ctx* x, void* stream) {
  if (!x || x->cfg.n_experts == 0) return SPECDEC_E_INVAL;
  HIP_TRY(launch_fill_i32(at<int>(x, x->lay.e_usage), 0, (size_t)x->cfg.n_layers,
                          reinterpret_cast<hipStream_t>(stream)));
  x->moe_usage_on = true;
  return SPECDEC_OK;
}

int specdec_moe_usage_read(specdec_ctx* x, int32_t* per_layer, void* stream) {
  if (!x || !per_layer || x->cfg.n_experts == 0) return SPECDEC_E_INVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(hipMemcpyAsync(per_layer, at<int>(x, x->lay.e_usage), (size_t)x->cfg.n_layers * 4,
                         hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  x->moe_usage_on = false;
  return SPECDEC_OK;
}

int specdec_profile_start(specdec_ctx* x, int32_t cls, int32_t capacity) {
  if (!x || capacity < 0 || cls < -1 || cls > 8) return SPECDEC_E_INVAL;
  for (auto e : x->prof_ev) (void)hipEventDestroy(e);
  x->prof_ev.clear();
  x->prof_class = -1;
  x->prof_n = 0;
  x->prof_cap = 0;
  x->prof_ev.resize((size_t)2 * capacity);
  for (auto& e : x->prof_ev) HIP_TRY(hipEventCreate(&e));
  x->prof_cap = capacity;
  x->prof_class = cls;
  return SPECDEC_OK;
}

int specdec_profile_read(specdec_ctx* x, float* ms_out, int32_t max, int32_t* n_out) {
  if (!x || !n_out) return SPECDEC_E_INVAL;
  const int n = std::min(x->prof_n, max);
  for (int i = 0; i < n; ++i) {
    HIP_TRY(hipEventSynchronize(x->prof_ev[2 * i + 1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, x->prof_ev[2 * i], x->prof_ev[2 * i + 1]));
    if (ms_out) ms_out[i] = ms;
  }
  *n_out = n;
  x->prof_class = -1;
  return SPECDEC_OK;
}

int specdec_query_split(specdec_ctx* x, int32_t cls, int32_t* splits, int32_t* units,
                        int32_t* waves, int32_t* groups) {
  if (!x || !splits || !units || !waves || !groups) return SPECDEC_E_INVAL;
  const Gemm* g = nullptr;
  switch (cls) {
    case 0: g = &x->g_gu[0]; break;
    case 1: g = &x->g_down[0]; break;
    case 2: g = &x->g_qkv[0]; break;
    case 3: g = &x->g_o[0]; break;
    case 5: g = &x->g_head; break;
    case 7: if (x->g_egu.empty()) return SPECDEC_E_INVAL; g = &x->g_egu[0]; break;
    case 8: if (x->g_edown.empty()) return SPECDEC_E_INVAL; g = &x->g_edown[0]; break;
    default: return SPECDEC_E_INVAL;
  }
  *splits = g->KW;
  *units = g->n_units;
  *waves = g->NW;
  *groups = cdiv(g->n_units, g->NW / g->KW);
  return SPECDEC_OK;
}

int specdec_query_launch(specdec_ctx* x, int32_t cls, int32_t rows, int32_t* splits,
                         int32_t* tiles_per_unit, int32_t* units, int32_t* waves, int32_t* groups) {
  if (!x || !tiles_per_unit || rows < 1 || rows > x->cfg.max_batch * x->cfg.max_rows)
    return SPECDEC_E_INVAL;
  int rc = specdec_query_split(x, cls, splits, units, waves, groups);
  if (rc) return rc;
  const Gemm* g = nullptr;
  switch (cls) {
    case 0: g = &x->g_gu[0]; break;
    case 1: g = &x->g_down[0]; break;
    case 2: g = &x->g_qkv[0]; break;
    case 3: g = &x->g_o[0]; break;
    case 5: g = &x->g_head; break;
    case 7: g = &x->g_egu[0]; break;
    default: g = &x->g_edown[0]; break;
  }
  GemmArgs a;
  a.nu = g->NU;
  a.n_units = g->n_units;
  a.NW = g->NW;
  if (cls == 0) wide_units(a, *g, rows);
  *tiles_per_unit = a.nu;
  *units = a.n_units;
  *waves = a.NW;
  *groups = cdiv(a.n_units, a.NW / g->KW);
  return SPECDEC_OK;
}

const char* specdec_error_string(int code) {
  switch (code) {
    case SPECDEC_OK: return "ok";
    case SPECDEC_E_INVAL: return "invalid argument";
    case SPECDEC_E_CAPACITY: return "KV-cache capacity exceeded";
    case SPECDEC_E_HIP: return "HIP launch failure";
    case SPECDEC_E_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown error";
  }
}

}  // extern "C"
