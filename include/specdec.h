/*
 * libspecdec -- greedy speculative decoding with a multi-token-prediction (MTP) drafter on one
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The step (sources are five web pages on Gemma 4's MTP drafters):
 *   1. specdec_draft     -- a light drafter head reads the target's last hidden state and
 *                           cross-attends to the target's own KV cache (it keeps no cache), then
 *                           proposes K tokens autoregressively through a clustered output layer
 *                           ("Accelerating Gemini Nano on Pixel with frozen multi-token
 *                           prediction", sections "The 'late exit' strategy" and "Zero-copy
 *                           architecture"; "Gemma 4's MTP drafter explained", section "What is
 *                           different about Gemma 4's drafter?").
 *   2. specdec_verify    -- the target runs one forward pass over the current token and the K
 *                           drafts ("Gemma 4's MTP drafter explained", section "How does
 *                           speculative decoding work?").
 *   3. specdec_accept    -- drafts are accepted up to the first disagreement, the rest dropped,
 *                           and the target's own token appended: 1..K+1 tokens per step (same
 *                           section; "Accelerating Gemma 4 ...", section "How MTP works").
 *   4. specdec_kv_commit -- the cache rolls back to the first mismatch: only the committed
 *                           length moves; dead entries are overwritten by the next verify
 *                           ("Accelerating Gemini Nano on Pixel ...", "The 'late exit' strategy").
 *
 * Conventions for every call:
 *   - All device buffers are allocated and owned by the caller.  The library never allocates
 *     or frees device memory and never synchronises the stream in the step calls; every step
 *     call only enqueues kernels on `stream` (a hipStream_t passed as void*; NULL = default).
 *   - Return value: SPECDEC_OK (0) or a negative SPECDEC_E_* code; on error nothing has been
 *     enqueued unless the code is SPECDEC_E_HIP (a launch failed part-way).
 *   - Kernels never write out of bounds.  Conditions only visible on the device (a cache slot
 *     beyond max_ctx, an out-of-range token id, a NaN logit) set bits in a sticky device error
 *     word read with specdec_read_device_error.
 *   - One context serves one stream / host thread at a time.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPECDEC_OK = 0,
  SPECDEC_E_INVAL = -1,       /* null pointer, bad shape, B/K/rows beyond the configured maxima */
  SPECDEC_E_CAPACITY = -2,    /* host-side bound on len + rows exceeds max_ctx */
  SPECDEC_E_HIP = -3,         /* a HIP launch / runtime call failed */
  SPECDEC_E_UNSUPPORTED = -4  /* configuration the kernels are not built for */
};

enum { SPECDEC_F32 = 0, SPECDEC_BF16 = 1 };
enum { SPECDEC_HEAD_CLUSTERED = 0, SPECDEC_HEAD_FULL = 1 };
enum { SPECDEC_WF_DENSE = 0, SPECDEC_WF_Q4 = 1 };
#define SPECDEC_ACCEPT_COMMIT 1u

/* Device error word bits. */
enum { SPECDEC_DEVERR_CAPACITY = 1, SPECDEC_DEVERR_NAN = 2, SPECDEC_DEVERR_TOKEN = 4 };

/* Packing kinds for specdec_pack_matrix. */
enum {
  SPECDEC_PACK_PLAIN = 0,   /* any projection */
  SPECDEC_PACK_ROPE = 1,    /* rows are heads of head_dim whose rotary pairs (i, i+hd/2) are
                               made adjacent: the fused q/k/v projection and the drafter's q */
  SPECDEC_PACK_GATE_UP = 2  /* rows [0,F) gate and [F,2F) up, interleaved per 16-row tile */
};

typedef struct {
  /* target decoder (pre-norm RMSNorm, RoPE, gated SiLU FFN, tied LM head) */
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  /* mixture of experts: n_experts == 0 means a dense FFN of ffn_dim; otherwise each layer's FFN
     is the weighted sum of its top_k of n_experts gated experts of width expert_ffn plus a
     shared gated FFN of width shared_ffn (ffn_dim unused) */
  int32_t n_experts, top_k, expert_ffn, shared_ffn;
  /* drafter: d_layers layers of width d_dim, FFN d_ffn, n_centroids equal clusters of the
     vocabulary, cross-attending to target layer kv_src_layer (-1 = last) */
  int32_t d_layers, d_dim, d_ffn, n_centroids, kv_src_layer;
  int32_t dtype;            /* SPECDEC_F32 | SPECDEC_BF16: weights, KV and GEMM inputs */
  float rms_eps, rope_theta;
  int32_t max_batch;        /* sequences per call */
  int32_t max_draft;        /* largest K */
  int32_t max_rows;         /* largest rows per sequence in one verify (>= max_draft + 1) */
  int32_t max_ctx;          /* KV-cache positions per sequence */
  int32_t weight_format;    /* SPECDEC_WF_DENSE: packed matrices hold dtype elements;
                               SPECDEC_WF_Q4: every packed matrix (target, drafter, embedding,
                               table, centroids) is in the 4-bit block format of
                               specdec_pack_q4; needs dtype BF16 and every reduction width
                               (d_model, Hq*hd, the FFN widths, d_dim, d_ffn) % 128 == 0 */
  int32_t max_prefill;      /* rows of the largest specdec_prefill call, 0..1024 (0: none).  Above
                               0 it needs dtype BF16, no experts, d_model, Hq*hd, ffn_dim % 64
                               == 0 and hd in {64, 128, 256}; the workspace grows by the chunk's
                               activations and 60 MiB of GEMM partials.  With 4-bit weights the
                               prompt GEMM rounds each weight d * (q - 8) to bf16 */
} specdec_config;

/* Per-layer tensor slots of specdec_weights.layers (n_layers * SPECDEC_N_LAYER_TENSORS). */
enum {
  SPECDEC_LW_ATTN_NORM = 0, /* float [d_model] */
  SPECDEC_LW_QKV = 1,       /* packed (ROPE) [Hq*hd + 2*Hkv*hd][d_model]: Wq rows, Wk rows, Wv rows */
  SPECDEC_LW_O = 2,         /* packed [d_model][Hq*hd] */
  SPECDEC_LW_FFN_NORM = 3,  /* float [d_model] */
  SPECDEC_LW_GATE_UP = 4,   /* packed (GATE_UP) [2*F][d_model], F = ffn_dim (dense) or
                               shared_ffn (the shared FFN of a mixture-of-experts layer) */
  SPECDEC_LW_DOWN = 5,      /* packed [d_model][F] */
  /* mixture-of-experts layers only (NULL for a dense model): */
  SPECDEC_LW_ROUTER = 6,    /* packed [n_experts][d_model] */
  SPECDEC_LW_EXP_GATE_UP = 7, /* n_experts packed (GATE_UP) [2*expert_ffn][d_model] matrices,
                                 back to back in expert order */
  SPECDEC_LW_EXP_DOWN = 8,  /* n_experts packed [d_model][expert_ffn] matrices, back to back */
  SPECDEC_N_LAYER_TENSORS = 9
};

/* Per-layer tensor slots of specdec_weights.d_layers (d_layers * SPECDEC_N_DRAFT_TENSORS). */
enum {
  SPECDEC_DW_N1 = 0,        /* float [d_dim] */
  SPECDEC_DW_Q = 1,         /* packed (ROPE) [Hq*hd][d_dim] */
  SPECDEC_DW_O = 2,         /* packed [d_dim][Hq*hd] */
  SPECDEC_DW_N2 = 3,        /* float [d_dim] */
  SPECDEC_DW_GATE_UP = 4,   /* packed (GATE_UP) [2*d_ffn][d_dim] */
  SPECDEC_DW_DOWN = 5,      /* packed [d_dim][d_ffn] */
  SPECDEC_N_DRAFT_TENSORS = 6
};

/* Device pointers to the weights (dtype elements unless noted).  "packed" tensors are in the
   streaming tile layout written by specdec_pack_matrix (weight_format SPECDEC_WF_DENSE) or in
   the 4-bit block format written by specdec_pack_q4 (SPECDEC_WF_Q4).  The pointer tables are copied at
   create; the tensors themselves must outlive the context. */
typedef struct {
  const void* embed;             /* packed [vocab][d_model]; also the tied LM head */
  const float* final_norm;       /* [d_model] */
  const void* const* layers;     /* n_layers * SPECDEC_N_LAYER_TENSORS pointers */
  const void* table;             /* packed [vocab][d_dim], cluster-major rows (tied drafter
                                    input embedding and output table) */
  const void* centroids;         /* packed [n_centroids][d_dim] */
  const int32_t* row_vocab;      /* [vocab]: vocabulary id of table row r */
  const int32_t* vocab_row;      /* [vocab]: table row of vocabulary id v */
  const float* norm_h;           /* [d_model] drafter norm of the target hidden input */
  const float* norm_e;           /* [d_dim]   drafter norm of the token embedding input */
  const void* w_in;              /* packed [d_dim][d_model + d_dim] */
  const void* const* d_layers;   /* d_layers * SPECDEC_N_DRAFT_TENSORS pointers */
  const float* norm_f;           /* [d_dim] drafter final norm */
  const void* w_back;            /* packed [d_model][d_dim]: drafter state -> next hidden input */
} specdec_weights;

typedef struct specdec_ctx specdec_ctx; /* host memory; owns no device memory */

/* Bytes of device workspace a context with this configuration needs (0 if the config is
   invalid).  Size = f(config) only. */
size_t specdec_workspace_bytes(const specdec_config* cfg);

/* Elements of the KV cache per tensor (K or V): n_layers*max_batch*n_kv_heads*max_ctx*head_dim.
   K element (l, b, g, pos, c) sits at (((l*max_batch + b)*n_kv_heads + g)*max_ctx + pos)*head_dim + c;
   V is stored transposed per head: (((l*max_batch + b)*n_kv_heads + g)*head_dim + c)*max_ctx + pos,
   so that both attention operands stream along their reduction axis. */
size_t specdec_kv_elems(const specdec_config* cfg);

/* Creates a context over caller-owned device memory:
     kv_k, kv_v  [n_layers][max_batch][n_kv_heads][max_ctx][head_dim] dtype
     len         int32 [max_batch]: committed KV length per sequence (device-resident state)
     hid         float [max_batch][d_model]: the drafter's hidden input (the target's
                 pre-final-norm residual of the last committed position)
     workspace   specdec_workspace_bytes(cfg) bytes, 256-byte aligned
   Enqueues two small kernels on `stream`: one zeroes the device error word, one tabulates the
   rotary (cos, sin) of every position in the workspace.  Errors: SPECDEC_E_INVAL (null pointers, shapes not multiples of the
   tile: d_model, Hq*hd, ffn_dim (dense), expert_ffn and shared_ffn (MoE), d_dim, d_ffn % 32;
   head_dim % 16, head_dim <= 256; vocab % 64; vocab / n_centroids % 64; n_centroids % 16;
   max_batch*max_rows <= 64; max_rows <= 64; max_ctx % 8; MoE: n_experts <= 256 and % 16,
   1 <= top_k <= min(16, n_experts)), SPECDEC_E_UNSUPPORTED (head_dim not one of 64, 128,
   176, 256). */
int specdec_create(const specdec_config* cfg, const specdec_weights* w, void* kv_k, void* kv_v,
                   int32_t* len, float* hid, void* workspace, size_t workspace_bytes,
                   void* stream, specdec_ctx** out);
/* For callers that cannot allocate device memory (code under stream capture, serving loops or
   harnesses that forbid hipMalloc): specdec_create with the workspace taken from a fixed array
   of SPECDEC_STATIC_WORKSPACE_BYTES inside the library instead of a caller buffer.  Each GPU the
   library runs on holds its own copy of the array until the process ends; its address is looked
   up (hipGetSymbolAddress) on the first call on that GPU, with that GPU current.  This call
   allocates nothing: the caller still owns kv_k, kv_v, len and hid, as for specdec_create.
   Every context made by this call on one GPU shares that GPU's array, which keeps what the last
   call left there: use one such context per GPU at a time (creating another takes the array
   over), and calls on it that overlap on one GPU race.  Create zeroes the device error word and
   writes the rotary table there, as specdec_create does in its workspace; every other part of
   the workspace is written by a step before it is read.
   Errors: those of specdec_create, and SPECDEC_E_CAPACITY when specdec_workspace_bytes(cfg)
   exceeds SPECDEC_STATIC_WORKSPACE_BYTES (checked before any HIP call). */
#define SPECDEC_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int specdec_create_static(const specdec_config* cfg, const specdec_weights* w, void* kv_k,
                          void* kv_v, int32_t* len, float* hid, void* stream, specdec_ctx** out);

int specdec_destroy(specdec_ctx* ctx);

/* Draft K tokens per sequence.
   Inputs: cur_tok int32 [B] (device): the current token c0 at position len[b], not yet in the
   cache; hid (context state) and the target's layer-kv_src_layer cache, keys [0, len[b]).
   Sub-step j = 1..K embeds c_{j-1}, runs the drafter at query position len[b]+j-1 and scores
   the head: SPECDEC_HEAD_CLUSTERED scores the n_centroids centroids, keeps the k_c best
   clusters (ties -> lower cluster id) and takes the argmax over their member tokens;
   SPECDEC_HEAD_FULL scores the whole vocabulary (the fallback that drops the clusters).
   Ties -> lower vocabulary id.  Output drafts int32 [B][K] (device).
   Optional workload injection (tests and benchmarks; NULL = off): inject int32 [B][inj_stride]
   (device); entry (len[b]+j)*K + (j-1) >= 0 replaces draft j after it was drafted (the drafter's
   own token still feeds sub-step j+1).  Optional verify_tokens int32 [B][K+1] (device; NULL =
   skip) receives the next verify's input rows [c0, d1..dK] (drafts after injection), so a batch
   goes from draft to verify without a copy; it may overlap cur_tok at column 0.
   Errors: SPECDEC_E_INVAL (B > max_batch, K < 1, K > max_draft, k_c outside [1, n_centroids],
   null pointers), SPECDEC_E_CAPACITY (the host-side bound of len + K exceeds max_ctx: the last
   sub-step's query position len + K - 1 must be a cache slot). */
int specdec_draft(specdec_ctx* ctx, int32_t B, int32_t K, int32_t head_mode, int32_t k_c,
                  const int32_t* cur_tok, int32_t* drafts, const int32_t* inject,
                  int64_t inj_stride, int32_t* verify_tokens, void* stream);

/* What one drafting call can report besides its tokens, per sequence b and sub-step j (tests and
   measurement; every pointer is device memory and may be NULL to skip that part):
     state           float [B][K][d_dim]: the head's input s = rms(x) * norm_f of sub-step j
     hidden          float [B][K][d_model]: the next sub-step's hidden input W_back . s
     centroid_scores float [B][K][n_centroids]: the centroid scores C . s (clustered head only)
     table_scores    float [B][K][vocab], by table row (cluster-major, row_vocab maps a row to
                     its vocabulary id): only the rows the head scored are written (the members of
                     the selected clusters, or every row for the full head); the caller fills the
                     buffer first with a value it can tell apart (NaN)
     raw_drafts      int32 [B][K]: the drafter's own token of sub-step j, before injection
   The same kernels run with or without a trace; a trace only adds copies after them. */
typedef struct {
  float* state;
  float* hidden;
  float* centroid_scores;
  float* table_scores;
  int32_t* raw_drafts;
} specdec_draft_trace;

/* specdec_draft with an optional trace (NULL = none, which is specdec_draft). */
int specdec_draft_traced(specdec_ctx* ctx, int32_t B, int32_t K, int32_t head_mode, int32_t k_c,
                         const int32_t* cur_tok, int32_t* drafts, const int32_t* inject,
                         int64_t inj_stride, int32_t* verify_tokens,
                         const specdec_draft_trace* trace, void* stream);

/* Target forward over n_rows rows per sequence: tokens int32 [B][n_rows] (device) at positions
   len[b] .. len[b]+n_rows-1.  Row i attends keys [0, len[b]+i].  Appends the rows' keys and
   values to the cache tentatively (len is not changed).  Keeps per-row hidden states and LM-head
   argmax partials in the workspace for specdec_accept / specdec_kv_commit.
   Optional outputs (NULL = skip): logits float [B][n_rows][vocab], argmax int32 [B][n_rows].
   Prefill is verify(n_rows = chunk) + kv_commit(chunk) per chunk.
   Errors: SPECDEC_E_INVAL (B, n_rows out of range), SPECDEC_E_CAPACITY (the host-side upper
   bound of len + n_rows exceeds max_ctx). */
int specdec_verify(specdec_ctx* ctx, int32_t B, int32_t n_rows, const int32_t* tokens,
                   float* logits, int32_t* argmax, void* stream);

/* ---- Token trees: several drafted continuations verified in one target pass ----
   Standard speculative decoding bets on one future path; the pages describe letting the drafter
   explore branching possibilities in parallel so that a long sequence is accepted more often in
   uncertain contexts ("Accelerating Gemini Nano on Pixel with frozen multi-token prediction",
   section "Future directions").  A tree has n_nodes <= max_rows nodes in topological order given
   by a host array parent[n_nodes]: parent[0] = -1 (the root: the current token, not yet in the
   cache) and 0 <= parent[i] < i; the depth of a node (its parent's plus one) is at most
   SPECDEC_TREE_MAX_DEPTH.  Node i of sequence b is the token at position len[b] + depth(i); during
   the verify its key and value sit in cache slot len[b] + i, and it attends to the committed
   prefix [0, len[b]) and the slots of its ancestors and itself. */
#define SPECDEC_TREE_MAX_DEPTH 16
#define SPECDEC_TREE_MAX_WIDTH 16

/* Drafts a tree of `width` branches of `depth` tokens per sequence: the first sub-step's `width`
   best tokens (highest score, then lower vocabulary id, among the tokens the head scores: the
   members of the k_c selected clusters, or the whole vocabulary) start the branches; each branch
   then continues greedily with its own tokens and hidden states (sub-step j of every branch reads
   the same committed keys [0, len) and queries at position len + j - 1).  Output tree_tokens int32
   [B][1 + width*depth] (device) in node order: node 0 = cur_tok, node 1 + width*(j-1) + k = the
   j-th token of branch k, whose parent is node 1 + width*(j-2) + k (j >= 2) or the root (j = 1).
   Optional injection (tests and benchmarks): entry (len[b] + j) * (width*depth) + (node - 1) of
   inject [B][inj_stride], when >= 0, replaces the node's token after drafting (the branch
   continues from its own token).  Errors: SPECDEC_E_INVAL (width or depth outside [1, 16],
   1 + width*depth > max_rows, B*width > max_batch*max_rows, bad head arguments, null pointers),
   SPECDEC_E_CAPACITY (the host-side bound of len + depth exceeds max_ctx). */
int specdec_draft_tree(specdec_ctx* ctx, int32_t B, int32_t width, int32_t depth, int32_t head_mode,
                       int32_t k_c, const int32_t* cur_tok, int32_t* tree_tokens,
                       const int32_t* inject, int64_t inj_stride, void* stream);

/* specdec_verify over the nodes of a tree: tokens int32 [B][n_nodes] (device), positions and
   visibility as described above; logits / argmax as for specdec_verify, per node.  Errors:
   SPECDEC_E_INVAL (a malformed tree, n_nodes > max_rows), SPECDEC_E_CAPACITY (host-side bound of
   len + n_nodes exceeds max_ctx). */
int specdec_verify_tree(specdec_ctx* ctx, int32_t B, int32_t n_nodes, const int32_t* parent,
                        const int32_t* tokens, float* logits, int32_t* argmax, void* stream);

/* Acceptance after specdec_verify_tree of the same tree: G[i] = argmax of node i (lowest id on
   ties); the accepted path is the longest root path on which every node's token equals G at its
   parent (among equally long ones, the lower node index at the first place they differ);
   out_tokens[b] (int32 [B][out_ld], out_ld >= tree depth + 1) = the tokens of its m nodes, then
   G at its last node, then -1; n_emit[b] = m + 1; next_tok[b] = G at
   the last node.  With SPECDEC_ACCEPT_COMMIT also len[b] += m + 1, hid[b] = hidden of the last
   node, and the path's cache entries are moved to slots len + 1 .. len + m (in every layer), so
   the cache again holds exactly the accepted sequence.  Errors: SPECDEC_E_INVAL (a different
   tree or batch than the last verify, out_ld too small, null pointers). */
int specdec_accept_tree(specdec_ctx* ctx, int32_t B, int32_t n_nodes, const int32_t* parent,
                        const int32_t* tokens, int32_t* out_tokens, int32_t out_ld,
                        int32_t* n_emit, int32_t* next_tok, uint32_t flags, void* stream);

/* Acceptance after a verify of K+1 rows per sequence (tokens = [c0, d1..dK], the verify input).
   One fused kernel per call: G[i] = argmax of row i (lowest id on ties); m = largest j <= K with
   tokens[1..j] == G[0..j-1]; out_tokens[b] = tokens[1..m], G[m], then -1 padding (int32
   [B][K+1]); n_emit[b] = m+1; next_tok[b] = G[m].  With SPECDEC_ACCEPT_COMMIT the same kernel
   also commits: len[b] += m+1 and hid[b] = hidden of row m.  Any output pointer may be NULL.
   Errors: SPECDEC_E_INVAL (K+1 != rows of the last verify, B != its batch, the last verify was a
   tree's). */
int specdec_accept(specdec_ctx* ctx, int32_t B, int32_t K, const int32_t* tokens,
                   int32_t* out_tokens, int32_t* n_emit, int32_t* next_tok, uint32_t flags,
                   void* stream);

/* Prompt prefill ("Gemma 4 MTP Drafter", section "How it works": the target first processes the
   prompt and the context; "Accelerating Gemini Nano on Pixel ...", section "Zero-copy
   architecture": the drafter then reads the target's cache and needs no prefill of its own).
   Runs T tokens (int32 [T], device) of sequence b (0 <= b < max_batch) through the target at
   positions len[b] .. len[b]+T-1, as one forward pass over the chunk (causal attention over the
   committed prefix and the chunk's earlier rows), appends their K/V, and commits them:
   len[b] += T, hid[b] = the pre-final-norm hidden state of the last row.  logits (fp32 [T][vocab],
   device) and argmax (int32 [T], device; argmax[T-1] is the first generated token) are optional.
   Uses the compute-bound prompt GEMM (weights read once per chunk, not once per row).  Cancels a
   pending verify (its accept / kv_commit are refused afterwards).  Errors: SPECDEC_E_INVAL,
   SPECDEC_E_CAPACITY (len[b] + T beyond max_ctx on the host-side bound), SPECDEC_E_UNSUPPORTED
   (max_prefill == 0). */
int specdec_prefill(specdec_ctx* ctx, int32_t b, int32_t T, const int32_t* tokens, float* logits,
                    int32_t* argmax, void* stream);

/* Commit n_commit[b] (int32 [B], device, 1..rows of the last verify) rows: len[b] += n and
   hid[b] = hidden of row n-1.  For prefill chunks and callers that decide acceptance
   themselves.  Errors: SPECDEC_E_INVAL. */
int specdec_kv_commit(specdec_ctx* ctx, int32_t B, const int32_t* n_commit, void* stream);

/* Packs a logical row-major matrix src [n][kd] (device, dtype) into the streaming tile layout
   dst (device, n*kd elements).  kind: SPECDEC_PACK_*; head_dim for ROPE; split_rows = F for
   GATE_UP: n = 2F, or n = G*2F for G stacked [2F][kd] matrices (experts: gate rows then up
   rows each), packed group by group.  Requires n % 16 == 0, kd % 32 == 0.  A plain stack of G
   [n/G][kd] matrices packs as one [n][kd] PLAIN matrix.  Setup-time helper. */
int specdec_pack_matrix(const void* src, void* dst, int32_t n, int32_t kd, int32_t dtype,
                        int32_t kind, int32_t head_dim, int32_t split_rows, void* stream);

/* 4-bit block weights ("Gemma 4's MTP drafter explained", section "Step 1 -- repackaging the
   QAT drafter": the QAT drafters and targets keep every 32-weight block of a matrix on a 4-bit
   grid, stored as Q4_0).  Logical weight (row i, column k) = step[i][k/32] * (code[i][k] - 8),
   code 0..15, step an IEEE fp16 value.
   specdec_pack_q4 writes the matrix given by codes [n][kd] (device, one byte per code, only the
   low 4 bits read) and steps [n][kd/32] (device, fp16 bit patterns) into dst (device,
   specdec_q4_bytes(n, kd) = n*kd*9/16 bytes, 256-byte aligned), rows permuted by kind,
   head_dim and split_rows exactly as specdec_pack_matrix does.  Requires n % 16 == 0,
   kd % 128 == 0.  Layout (for reference; the library reads it): 1152-byte blocks per 16 rows x
   128 columns, tile-major; a block holds 1024 bytes of codes (16 bytes per MFMA operand lane)
   and then each row's four fp16 steps.  Setup-time helper; errors: SPECDEC_E_INVAL. */
size_t specdec_q4_bytes(int32_t n, int32_t kd);
int specdec_pack_q4(const uint8_t* codes, const uint16_t* steps, void* dst, int32_t n, int32_t kd,
                    int32_t kind, int32_t head_dim, int32_t split_rows, void* stream);

/* Tightens the host-side bound on len after the caller has read len back (host values). */
int specdec_set_len_bound(specdec_ctx* ctx, const int32_t* host_len, int32_t B);

/* Reads (synchronously) and optionally clears the sticky device error word. */
int specdec_read_device_error(specdec_ctx* ctx, int32_t* host_word, int32_t clear, void* stream);

/* Per-launch timing of one kernel class, for roofline reporting: after specdec_profile_start,
   every launch of that class is timed (up to `capacity` launches), a single-kernel GEMM launch by
   HIP events attached to its own dispatch, the others by events recorded on the launch stream
   around their kernels.  specdec_profile_read synchronises and returns the durations in ms.
   Classes: 0 gate/up GEMM, 1 down GEMM, 2 qkv GEMM, 3 o GEMM, 4 attention, 5 LM head,
   6 drafter head, 7 routed-expert gate/up GEMM, 8 routed-expert down GEMM.  Not for use under
   graph capture. */
int specdec_profile_start(specdec_ctx* ctx, int32_t kernel_class, int32_t capacity);
int specdec_profile_read(specdec_ctx* ctx, float* ms_out, int32_t max, int32_t* n_out);

/* Mixture-of-experts measurement: specdec_moe_usage_start zeroes per-layer counters (enqueued on
   `stream`) and from then on each verify adds, per layer, the number of distinct experts its rows
   were routed to (the experts whose weights it read).  specdec_moe_usage_read synchronises
   `stream`, copies the n_layers counters to host memory and stops counting.  Errors:
   SPECDEC_E_INVAL for a dense model or null pointers. */
int specdec_moe_usage_start(specdec_ctx* ctx, void* stream);
int specdec_moe_usage_read(specdec_ctx* ctx, int32_t* per_layer, void* stream);

/* Launch shape the context uses for a GEMM class (classes 0, 1, 2, 3, 5 above; tests and
   reports; classes 7, 8 for a mixture-of-experts model): split-K factor, work units, waves per
   workgroup and workgroups of one launch (for 7 and 8: the upper bound, all experts). */
int specdec_query_split(specdec_ctx* ctx, int32_t kernel_class, int32_t* splits, int32_t* units,
                        int32_t* waves, int32_t* groups);

/* The same for a call of `rows` rows in all (1 <= rows <= max_batch * max_rows), which may take
   wider work units than the context's default (one per workgroup); also returns the 16-column
   tiles per unit.  A unit's split-K never depends on `rows`.  Errors: SPECDEC_E_INVAL for a bad class, row count or
   null pointer. */
int specdec_query_launch(specdec_ctx* ctx, int32_t kernel_class, int32_t rows, int32_t* splits,
                         int32_t* tiles_per_unit, int32_t* units, int32_t* waves, int32_t* groups);

/* Draft-length policy (host code, no device work): picks the next step's K from the running
   acceptance and the measured step costs.  The pages give the best draft length as a property of
   the hardware and the text (two drafted tokens on one consumer GPU, one on a slower one; more
   gain on predictable text): "Gemma 4's MTP drafter explained", sections "Tip: start with two
   drafted tokens" and "Why use a drafter?".
   Acceptance: a step that drafted K and emitted n (n_emit) accepted m = n - 1 drafts, and saw a
   disagreement iff m < K; the estimate is p = (A + a0) / (A + R + a0 + r0) with A, R the sums of
   m and of [m < K] over past steps, each decayed by `decay` per step, and a0, r0 the prior
   pseudo-counts.  Choice: the K in [k_min, k_max] maximising (1 + p + ... + p^K) /
   (K * t_draft_ms + t_verify_ms + K * t_row_ms), the smallest K on a tie.  t_draft_ms is one
   drafter sub-step, t_verify_ms a one-row verify (decode) step, t_row_ms each further row.
   The struct is caller memory; init fills every field. */
typedef struct {
  int32_t k_min, k_max;
  float decay, prior_accepted, prior_rejected;
  float t_draft_ms, t_verify_ms, t_row_ms;
  double accepted, rejected; /* decayed counts */
} specdec_k_policy;

/* Errors: SPECDEC_E_INVAL (k_min < 1, k_max < k_min, decay outside (0, 1], non-positive prior,
   negative or non-finite times, t_verify_ms <= 0). */
int specdec_k_policy_init(specdec_k_policy* pol, int32_t k_min, int32_t k_max, float decay,
                          float prior_accepted, float prior_rejected, float t_draft_ms,
                          float t_verify_ms, float t_row_ms);
/* Records one step that drafted K per sequence: n_emit (host int32 [B]) as specdec_accept
   returned it.  Errors: SPECDEC_E_INVAL (null, B < 1, K < 1, an n_emit outside [1, K+1]). */
int specdec_k_policy_observe(specdec_k_policy* pol, int32_t K, const int32_t* n_emit, int32_t B);
/* The current acceptance estimate p (-1 for a null policy). */
double specdec_k_policy_acceptance(const specdec_k_policy* pol);
/* The draft length for the next step (or SPECDEC_E_INVAL for a null policy). */
int32_t specdec_k_policy_choose(const specdec_k_policy* pol);

const char* specdec_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
