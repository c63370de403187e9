/*
 * medusa.h -- C ABI of the Medusa verify tree-step library for MI355X (gfx950).
 *
 * One verify tree-step of Medusa decoding, as the method is described in the
 * ICML 2024 paper summary "Medusa: Simple LLM Inference Acceleration Framework
 * with Multiple Decoding Heads" (section "基准/方法设计", the three components)
 * and the tutorial page "Medusa 多解码头推理加速全解析" (sections "推理算法"
 * and "超参数调优指南"):
 *
 *   (1) medusa_heads        K Medusa heads on the last hidden state
 *   (2) medusa_topk         per-head top-k over the vocabulary
 *       medusa_build_tree   candidate tree from a fixed list of rank paths
 *       medusa_tree_mask    its node arrays and ancestor bitmask
 *       medusa_tree_tokens  the token of every tree node
 *   (3) tree_attention      every node over the prefix KV cache + its ancestors
 *   (4) typical_accept      typical acceptance and the longest accepted prefix
 *       rejection_accept    the rejection-sampling rule it is compared with
 *   (5) medusa_kv_commit    append the accepted path to the KV cache
 *
 * Conventions (all calls):
 *  - Device buffers are plain device pointers owned by the caller; tensors are
 *    dense, row-major, in the layout given per argument.  Outputs must not
 *    alias inputs.  Token ids are int32.
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (uint16); f32 tensors hold
 *    float.  Device pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device calls only
 *    enqueue work; they never synchronise and never allocate device memory.
 *    Scratch memory is passed in as `ws`/`ws_bytes`, sized by the matching
 *    *_workspace call.
 *  - Every argument is checked before anything is launched.  On a non-OK
 *    status nothing has been enqueued and outputs are untouched;
 *    medusa_last_error() returns a thread-local description.  A failed launch
 *    returns MEDUSA_ERR_HIP.  Faults inside kernels surface at the caller's
 *    next synchronisation.  No C++ exception crosses this interface.
 *
 * Debug environment variables (read by the device calls; off by default):
 *  - MEDUSA_VALIDATE=1: before their kernels, medusa_topk and
 *    medusa_topk_tree_tokens[_tmax] check the logits for NaN and the root tokens
 *    for ids outside [0, V); typical_accept and rejection_accept check their
 *    logits for NaN and +inf and the tree tokens for ids outside [0, V).  A
 *    finding returns MEDUSA_ERR_NONFINITE (logits) or MEDUSA_ERR_ARG (ids)
 *    and enqueues nothing else, so the outputs are untouched.  The check is
 *    one extra kernel plus a synchronisation of `stream`, so it is refused
 *    (MEDUSA_ERR_STATE) while the stream is being captured into a graph.
 *    Without it, NaN logits give unspecified results, an out-of-range
 *    candidate token is never accepted, and an out-of-range root token is
 *    copied as it is.
 *  - MEDUSA_FAULT=launch: every kernel launch fails before it is enqueued;
 *    the call returns MEDUSA_ERR_HIP with nothing enqueued (error-path tests).
 *  - MEDUSA_TRACE=1: each device call is wrapped in a roctx range of its
 *    name (rocprofv3 --marker-trace); roctx is opened at run time.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEDUSA_ABI_VERSION 1

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_ARG = 1,          /* NULL / misaligned pointer, bad scalar argument   */
  MEDUSA_ERR_SHAPE = 2,        /* sizes that disagree with each other or the tree   */
  MEDUSA_ERR_TREE = 3,         /* path list that is not a valid candidate tree      */
  MEDUSA_ERR_UNSUPPORTED = 4,  /* valid request outside the supported limits        */
  MEDUSA_ERR_WORKSPACE = 5,    /* workspace smaller than the *_workspace size       */
  MEDUSA_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed        */
  MEDUSA_ERR_STATE = 7,        /* tree not uploaded to the device; validate mode    */
                               /* asked for under graph capture                     */
  MEDUSA_ERR_NONFINITE = 8     /* NaN (or, for acceptance, +inf) logits; reported   */
                               /* only with MEDUSA_VALIDATE=1                       */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

typedef void *medusa_stream_t;            /* a hipStream_t */
typedef struct medusa_tree medusa_tree;   /* opaque candidate tree */

/* Limits checked by the calls below. */
#define MEDUSA_MAX_TOPK 64        /* k of medusa_topk                         */
#define MEDUSA_MAX_TREE 1024      /* tree tokens T, root included             */
#define MEDUSA_MAX_HEADS_M 32     /* most rows of the weight-streaming kernel */

const char *medusa_last_error(void);      /* thread-local text of the last non-OK status */
int medusa_abi_version(void);

/* ------------------------------------------------------------------------- */
/* (1) Medusa heads.  Paper summary, section "基准/方法设计", first component:
 *     head k (0-based; it predicts the token k+2 places ahead of the last
 *     accepted one) is the one-layer ResBlock r = h + SiLU(W1_k h) followed
 *     by the vocabulary projection W2_k r; W1 = 0 reproduces the backbone's
 *     LM head exactly.  SiLU(x) = x * sigmoid(x).  No biases.
 *
 *  dt = MEDUSA_BF16: h, W1, W2, r are bf16; products accumulate in fp32 on
 *                    the matrix cores; r is rounded to bf16 (nearest-even).
 *  dt = MEDUSA_F32 : everything fp32.
 *  h      [M][H]       device, dt       last hidden state, one row per sequence
 *  W1     [K][H][H]    device, dt       row = output feature
 *  W2     [K][V][H]    device, dt       row = vocabulary entry
 *  r      [K][M][H]    device, dt       output of medusa_head_resblock
 *  logits [K][M][V]    device, float    output
 *  Limits: H % 128 == 0 for bf16 (H % 4 == 0 for f32); 1 <= M.  bf16 with
 *  M <= MEDUSA_MAX_HEADS_M (decode: one row per sequence) streams the weights
 *  once; larger M (the verify-pass shape, every tree node of every sequence,
 *  M = B*T; or the backbone LM head over those rows, a head with W1 = 0) runs
 *  a block-tiled matrix-core GEMM, which needs one head's weights and one
 *  head's M x H activations to span less than 4 GiB each.
 *  Errors: ERR_ARG (NULL, misaligned), ERR_UNSUPPORTED (H, 4 GiB), ERR_HIP.
 */
medusa_status medusa_head_resblock(medusa_stream_t stream, medusa_dtype dt, int K, int M, int H,
                                   const void *h, const void *W1, void *r);
medusa_status medusa_head_vocab(medusa_stream_t stream, medusa_dtype dt, int K, int M, int H,
                                int V, const void *r, const void *W2, float *logits);
/* both of the above, in order, on one stream */
medusa_status medusa_heads(medusa_stream_t stream, medusa_dtype dt, int K, int M, int H, int V,
                           const void *h, const void *W1, const void *W2, void *r,
                           float *logits);

/* Packed weights (bf16).  The same projections with W1 / W2 stored once,
 * ahead of decoding, in the matrix-core fragment order.  A fragment is the
 * 16 x 32 block of head k at row tile t (rows 16t..16t+15) and reduction step
 * s (columns 32s..32s+31), one contiguous 1 KiB block in lane order:
 *   frag[l][e] = W[k][16t + l % 16][32s + 8 (l / 16) + e],  l < 64, e < 8
 * (rows >= N zero).  The fragments of `group` consecutive row tiles (group =
 * 1, 2, 4 or 8) are interleaved step by step: within head k, fragment (t, s)
 * is number ((t / group) * (H / 32) + s) * group + t % group, and each head
 * holds ceil(N / 128) * 8 row tiles.  group = 1 keeps every tile's steps
 * contiguous and streams fastest to calls of up to 8 rows; group = 8 streams
 * fastest to 9 and more rows (measured on MI355X);
 * medusa_pack_group_for_rows(M) returns that choice.  The *_packed calls take
 * the group Wp was packed with.
 *  medusa_packed_weight_bytes: size of Wp for W [K][N][H] (0 if H % 32 != 0),
 *                       the same for every group.
 *  medusa_pack_weights: W [K][N][H] bf16 (device) -> Wp (device, caller-owned,
 *                       medusa_packed_weight_bytes bytes); needs H % 128 == 0;
 *                       ERR_ARG for a group outside {1, 2, 4, 8}.
 *  *_packed: as the calls above with dt = MEDUSA_BF16 and W1p = pack(W1)
 *            (N = H), W2p = pack(W2) (N = V). */
size_t medusa_packed_weight_bytes(int K, int N, int H);
int medusa_pack_group_for_rows(int M);
medusa_status medusa_pack_weights(medusa_stream_t stream, int K, int N, int H, int group, const void *W,
                                  void *Wp);
medusa_status medusa_head_resblock_packed(medusa_stream_t stream, int K, int M, int H, int group,
                                          const void *h, const void *W1p, void *r);
medusa_status medusa_head_vocab_packed(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                       const void *r, const void *W2p, float *logits);
medusa_status medusa_heads_packed(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                  const void *h, const void *W1p, const void *W2p, void *r, float *logits);

/* medusa_head_vocab_packed that also writes, for medusa_topk_tree_tokens_tmax,
 * the image of each 16-value tile's largest logit:
 *   tile_max [K][M][ceil(V/16)] device uint32 (output, 4-byte aligned),
 *   tile_max[k][m][t] = max of image(logits[k][m][v]) over v in
 *   [16t, min(16t + 16, V)),
 * where image(x) is the order-preserving map of the float's bits (-0.0 taken
 * as +0.0; the sign bit set for x >= +0, every bit inverted for x < 0), so
 * that images order as the values do.  The logits are bit-identical to
 * medusa_head_vocab_packed's.  M <= MEDUSA_MAX_HEADS_M (ERR_UNSUPPORTED
 * beyond); other errors as medusa_head_vocab_packed. */
medusa_status medusa_head_vocab_packed_tmax(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                            const void *r, const void *W2p, float *logits, uint32_t *tile_max);

/* Workspace variants of the packed calls, for many rows (the verify-pass
 * shape M = B*T, and the backbone's LM head over the tree nodes).  Same
 * arguments and results as medusa_head_resblock_packed /
 * medusa_head_vocab_packed (bit-identical: the same products, summed in the
 * same order), plus a caller-owned device workspace.  With M >= 65 the
 * activations (h, resp. r) are first copied into the workspace in the
 * fragment order of the packed weights (row tile of 16 rows x 32 columns as
 * one 1 KiB block in lane order), so that both operands of the block-tiled
 * matrix-core contraction stream as whole fragments; with M < 65 the calls
 * above run and ws is not touched (it may then be NULL).
 *  medusa_head_workspace(K, M, H): bytes of ws, K * ceil(M/16) * (H/32) KiB
 *                       for M >= 65 and H % 128 == 0, else 0.
 *  ws: device, 16-byte aligned, >= medusa_head_workspace(K, M, H) bytes
 *      (ERR_WORKSPACE if smaller); its contents on return are unspecified.
 *  Limits as the packed calls, and each head's packed activations < 4 GiB. */
size_t medusa_head_workspace(int K, int M, int H);
medusa_status medusa_head_resblock_packed_ws(medusa_stream_t stream, int K, int M, int H, int group,
                                             const void *h, const void *W1p, void *r, void *ws, size_t ws_bytes);
medusa_status medusa_head_vocab_packed_ws(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                          const void *r, const void *W2p, float *logits, void *ws,
                                          size_t ws_bytes);
/* Both of the above in one call (as medusa_heads_packed, bit-identical to it):
 * with M >= 65 the ResBlock also writes r in fragment order into the
 * workspace, and the vocabulary projection reads it there, so r is not copied
 * again.  r is still written row-major.
 *  medusa_heads_workspace(K, M, H): bytes of ws, (K + 1) * ceil(M/16) * (H/32)
 *                       KiB for M >= 65 and H % 128 == 0, else 0 (then ws may
 *                       be NULL).  Errors as the calls above. */
size_t medusa_heads_workspace(int K, int M, int H);
medusa_status medusa_heads_packed_ws(medusa_stream_t stream, int K, int M, int H, int V, int group, const void *h,
                                     const void *W1p, const void *W2p, void *r, float *logits, void *ws,
                                     size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* (2) Top-k of every row.  Tutorial page, sections "候选生成" and "每头 Top-K":
 *     each head contributes its top-k tokens.  Order: value descending, then
 *     token id ascending (-0.0 == +0.0); -inf allowed; NaN is not.
 *  logits [R][V] device float;  idx [R][k] device int32 (output);
 *  val    [R][k] device float (output, may be NULL): logits[r][idx].
 *  Limits: 1 <= k <= min(V, MEDUSA_MAX_TOPK); ceil(V/32768) * k <= 4096.
 *  ws: medusa_topk_workspace bytes (0 when V <= 32768, then ws may be NULL),
 *  8-byte aligned; calls that overlap in time must not share it.
 */
size_t medusa_topk_workspace(int R, int V, int k);
medusa_status medusa_topk(medusa_stream_t stream, int R, int V, int k, const float *logits,
                          int32_t *idx, float *val, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* Candidate trees (host calls).  Tutorial page, section "树结构：medusa_choices":
 * a tree is a list of rank paths; element d of a path is a rank within Medusa
 * head d's top-k.  Every proper prefix of a path must be in the list.
 *
 * Paths are passed flattened: ranks[p * K + d] for d < path_len[p] (entries
 * beyond path_len[p] are ignored).
 */

/* Dense tree (tutorial page, "候选生成": Cartesian product of the per-head
 * top-k): all sum_{d=1..K} k^d paths, depth then lexicographic order.
 * cap = capacity of path_len (ranks holds cap*K).  *n_paths receives the count. */
medusa_status medusa_dense_paths(int K, int k, int cap, int32_t *ranks, int32_t *path_len,
                                 int *n_paths);

/* Greedy sparse tree (paper summary, "方法细节": from per-head top-i accuracies,
 * repeatedly add the node with the largest expected gain in accept length).
 * acc[d * rank_cap + i] = accuracy of rank i of head d (host, K*rank_cap).
 * A node's gain is the product of acc along its path; equal gains (relative
 * difference below 1e-12) go to the shorter, then lexicographically smaller
 * path.  Writes n_paths paths in the order they were added. */
medusa_status medusa_greedy_paths(const double *acc, int K, int rank_cap, int n_paths,
                                  int32_t *ranks, int32_t *path_len);

/* Validate a path list and build the tree (host memory only).
 * Node 0 is the root (the greedy next token); node j >= 1 is the j-th path in
 * (length, lexicographic) order, so parents precede children.
 * ERR_TREE: length outside [1, K], rank outside [0, k), duplicate, or missing
 * prefix.  ERR_UNSUPPORTED: T = n_paths + 1 > MEDUSA_MAX_TREE or k > MEDUSA_MAX_TOPK.
 * The returned tree is owned by the caller (medusa_tree_free). */
medusa_status medusa_build_tree(const int32_t *ranks, const int32_t *path_len, int n_paths,
                                int K, int k, medusa_tree **out);

/* Node arrays of a tree (host outputs; every pointer may be NULL).
 *  T = tokens incl. root, W = ceil(T/64) mask words per row, depth_max, n_leaves;
 *  mask[T][W]: bit (i % 64) of word i/64 of row j set iff node i is j or one of
 *             j's ancestors (root included) -- paper summary, FAQ on tree
 *             attention: a token sees only the predecessors on its own branch;
 *  parent[T] (-1 for the root), depth[T], rank[T] (-1 for the root);
 *  retrieve[n_leaves][depth_max+1]: node ids root..leaf per leaf, -1 padded. */
medusa_status medusa_tree_mask(const medusa_tree *t, int *T, int *W, int *depth_max,
                               int *n_leaves, uint64_t *mask, int32_t *parent, int32_t *depth,
                               int32_t *rank, int32_t *retrieve);

/* Position of each tree token: L + depth (paper summary FAQ: positions follow
 * the tree structure).  pos: host [T]. */
medusa_status medusa_tree_positions(const medusa_tree *t, int L, int32_t *pos);

/* Copy the tree's arrays to the current HIP device (one allocation, synchronous).
 * Required once before the device calls that take the tree.  ERR_HIP on failure. */
medusa_status medusa_tree_upload(medusa_tree *t);

/* Free the host arrays and the device copy.  NULL is ignored. */
void medusa_tree_free(medusa_tree *t);

/* Token of every node: tree_tok[b][0] = root_tok[b],
 * tree_tok[b][j] = topk_idx[depth(j)-1][b][rank(j)]  (tutorial page, "候选生成":
 * a candidate is the base token followed by one choice per head).
 *  root_tok [B] device int32; topk_idx [K][B][k] device int32 (K >= depth_max,
 *  k > every rank in the tree); tree_tok [B][T] device int32 (output). */
medusa_status medusa_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B, int K,
                                 int k, const int32_t *root_tok, const int32_t *topk_idx,
                                 int32_t *tree_tok);

/* Both of the above in one pass: the per-head top-k of logits [K][B][V]
 * (written to topk_idx [K][B][k]) and the node tokens tree_tok [B][T], each
 * block that finishes a (head, sequence) row writing the tokens of the nodes
 * that row feeds.  ws: medusa_topk_workspace(K*B, V, k) bytes, as for medusa_topk. */
medusa_status medusa_topk_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B, int K, int V,
                                      int k, const float *logits, const int32_t *root_tok,
                                      int32_t *topk_idx, int32_t *tree_tok, void *ws, size_t ws_bytes);

/* medusa_topk_tree_tokens from tile maxima: tile_max [K][B][ceil(V/16)] is
 * what medusa_head_vocab_packed_tmax wrote together with these logits (with
 * any other contents the result is unspecified).  A row's top k lie in the
 * tiles whose image reaches a bound taken from the tile images, so each row
 * reads its tile images and then only those tiles instead of all V logits.
 * Outputs are identical to medusa_topk_tree_tokens'.  No workspace.  Errors
 * as medusa_topk_tree_tokens, plus ERR_UNSUPPORTED for V > 524288 or
 * K*B > 65535 and ERR_ARG for a NULL or misaligned tile_max. */
medusa_status medusa_topk_tree_tokens_tmax(medusa_stream_t stream, const medusa_tree *t, int B, int K, int V,
                                           int k, const float *logits, const uint32_t *tile_max,
                                           const int32_t *root_tok, int32_t *topk_idx, int32_t *tree_tok);

/* ------------------------------------------------------------------------- */
/* (3) Tree attention.  Paper summary, "基准/方法设计" (second component) and the
 *     FAQ on tree attention: all candidates share the prefix; node j attends
 *     to the L prefix positions and to the tree tokens on its own branch
 *     (its ancestors, the root and itself):
 *       out[b][j][h] = softmax(scale * q.[Kc ; Kt[anc(j)]]) . [Vc ; Vt[anc(j)]]
 *  dt = MEDUSA_BF16: bf16 in/out, scores/softmax/accumulation in fp32, the
 *                    probabilities enter the PV product as bf16;
 *  dt = MEDUSA_F32 : fp32 throughout.
 *  q, k_tree, v_tree  [B][T][nh][dh]  device, dt  (tree tokens, already position-encoded)
 *  k_cache, v_cache   [B][nh][L][dh]  device, dt  (the prefix cache; L may be 0)
 *  out                [B][T][nh][dh]  device, dt  (output)
 *  scale: 0 means 1/sqrt(dh).  Limits: dh in {64, 128}.
 *  ws: tree_attention_workspace bytes (split-prefix partial results).  The
 *  size, like the kernel chosen, depends on the current device's compute
 *  units: query it with the device current that the call will run on (a
 *  smaller workspace is refused with MEDUSA_ERR_WORKSPACE, never overrun). */
size_t tree_attention_workspace(medusa_dtype dt, const medusa_tree *t, int B, int nh, int dh,
                                int L);
medusa_status tree_attention(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t,
                             int B, int nh, int dh, int L, float scale, const void *q,
                             const void *k_tree, const void *v_tree, const void *k_cache,
                             const void *v_cache, void *out, void *ws, size_t ws_bytes);

/* Ragged prefixes (decode loop): the cache is [B][nh][L_cap][dh] and sequence
 * b attends to its first seq_len[b] cached keys (device int32 [B]; values
 * are clamped to [0, L_max]).  L_max <= L_cap is the host's bound on the
 * lengths and sizes the launch; ws: tree_attention_workspace(dt, t, B, nh,
 * dh, L_max) bytes.  Otherwise as tree_attention. */
medusa_status tree_attention_ragged(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t,
                                    int B, int nh, int dh, int L_cap, int L_max,
                                    const int32_t *seq_len, float scale, const void *q,
                                    const void *k_tree, const void *v_tree, const void *k_cache,
                                    const void *v_cache, void *out, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* (4) Typical acceptance.  Paper summary, "基准/方法设计" (third component) and
 *     "方法细节" (temperature): candidate token x at node c is kept if
 *       p(x) > min(eps, delta * exp(-H(p))),
 *     p = softmax(logits[b][parent(c)] / temperature), H its entropy (nats);
 *     the root is accepted greedily and unconditionally; a node counts only
 *     if its parent does; the longest accepted prefix wins, equal lengths
 *     going to the smallest node index.  temperature = 0 is greedy
 *     verification (p one-hot at the argmax).  eps = posterior_threshold,
 *     delta = posterior_alpha (tutorial page, "生成调用").
 *  logits   [B][T][V] device float  verification logits at every tree node
 *  tree_tok [B][T]    device int32
 *  accept_len [B]             device int32  accepted candidates after the root
 *  best_node  [B]             device int32  node that ends the accepted prefix
 *  next_tok   [B]             device int32  argmax (lowest id) of best's row
 *  accepted_tok [B][depth_max+1] device int32  tokens root..best, -1 padded
 *  cand_p, row_thr [B][T]     device float, optional (NULL): p of each node's
 *                             token under its parent, and each row's threshold
 *                             (nan where not evaluated).
 *  Limits: eps, delta >= 0; temperature >= 0.  ws: typical_accept_workspace
 *  bytes (the row pass's chunk partials, 32 bytes per sequence, node with
 *  children and 4096-wide chunk of V, then 16 bytes per sequence for the
 *  scan), 16-byte aligned. */
size_t typical_accept_workspace(const medusa_tree *t, int B, int V);
medusa_status typical_accept(medusa_stream_t stream, const medusa_tree *t, int B, int V,
                             const float *logits, const int32_t *tree_tok, float eps,
                             float delta, float temperature, int32_t *accept_len,
                             int32_t *best_node, int32_t *next_tok, int32_t *accepted_tok,
                             float *cand_p, float *row_thr, void *ws, size_t ws_bytes);

/* typical_accept without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (minus ws / ws_bytes) and results as
 * typical_accept (bit-identical: the same kernels).  The row pass's partials
 * go to a 4 MiB array the library keeps in each GPU's memory for the life of
 * the process (looked up on the first call on a device); the call allocates
 * nothing.  Limit: B * (number of tree nodes with children) * ceil(V / 4096)
 * + ceil(B / 2) <= 131072, else MEDUSA_ERR_UNSUPPORTED with nothing enqueued.  All calls on
 * one GPU share that array: calls that may overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller. */
medusa_status typical_accept_noalloc(medusa_stream_t stream, const medusa_tree *t, int B, int V,
                                     const float *logits, const int32_t *tree_tok, float eps, float delta,
                                     float temperature, int32_t *accept_len, int32_t *best_node,
                                     int32_t *next_tok, int32_t *accepted_tok, float *cand_p, float *row_thr);

/* (4b) Rejection-sampling acceptance, the rule typical acceptance replaces
 *     (paper summary, "两个扩展" and "关键发现"; the pages name it without
 *     spelling it out).  Starting at the root (always kept), the children of
 *     the current node u are tried in rank order: child c with token x is kept
 *     iff u_node[b][c] < min(1, p(x) / q(x)), p = softmax(logits[b][u] / T)
 *     (after the updates of the siblings rejected before c) and q =
 *     softmax(head_logits[depth(u)][b] / T), the head that drafted c; a
 *     rejected child replaces p by max(0, p - q) renormalised (kept as is if
 *     that is zero).  The first kept child becomes u.  With no child kept, or
 *     at a leaf, the next token is the inverse-CDF draw from the current p at
 *     u_bonus[b]: the smallest v with p(0) + ... + p(v) > u_bonus * sum(p).
 *     temperature 0: one-hot p and q at the argmax (lowest id) -- greedy
 *     verification.  Tokens outside [0, V) are never kept.
 *  logits      [B][T][V] device float   verification logits at every node
 *  head_logits [K][B][V] device float   the heads' logits (K >= depth_max)
 *  tree_tok    [B][T]    device int32
 *  u_node [B][T], u_bonus [B]  device float, uniforms in [0, 1) (u_node[b][0]
 *                              is not used)
 *  accept_len, best_node, next_tok [B], accepted_tok [B][depth_max+1]: as
 *  typical_accept.  keep_prob [B][T] device float, optional (NULL): the
 *  keep probability of every tried child, nan elsewhere.
 *  Errors: ERR_SHAPE (K < depth_max), ERR_ARG, ERR_UNSUPPORTED (V > 8 388 608). */
medusa_status rejection_accept(medusa_stream_t stream, const medusa_tree *t, int B, int V, int K,
                               const float *logits, const float *head_logits, const int32_t *tree_tok,
                               float temperature, const float *u_node, const float *u_bonus,
                               int32_t *accept_len, int32_t *best_node, int32_t *next_tok,
                               int32_t *accepted_tok, float *keep_prob);

/* ------------------------------------------------------------------------- */
/* (5) KV-cache commit.  Paper summary, "基准/方法设计" (the accepted prefix
 *     is kept and the next round starts after it) and tutorial page
 *     "部署与生成" (generation keeps the key/value cache): the K/V rows of
 *     the accepted path root..best_node[b] -- depth(best)+1 rows, in depth
 *     order -- are appended to sequence b's cache at positions
 *     seq_len[b] + depth (each node's tree position), then seq_len[b] grows
 *     by the rows written and, if next_tok / root_tok are given,
 *     root_tok[b] = next_tok[b] (the next step's root).
 *  k_tree, v_tree   [B][T][nh][dh]      device, dt
 *  best_node        [B]                 device int32 (typical_accept output)
 *  seq_len          [B]                 device int32, in/out
 *  k_cache, v_cache [B][nh][L_cap][dh]  device, dt, updated in place
 *  next_tok, root_tok [B]               device int32, both or neither (NULL)
 *  Rows that would pass L_cap are dropped (seq_len stops at L_cap); a
 *  sequence with best_node outside [0, T) or seq_len outside [0, L_cap] is
 *  left unchanged (its root is still advanced).  Needs dh * elem % 16 == 0. */
medusa_status medusa_kv_commit(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t, int B,
                               int nh, int dh, int L_cap, const void *k_tree, const void *v_tree,
                               const int32_t *best_node, int32_t *seq_len, void *k_cache,
                               void *v_cache, const int32_t *next_tok, int32_t *root_tok);

/* ------------------------------------------------------------------------- */
/* (6) Achievable peaks, for the roofline the step is reported against.  The
 *     paper summary ("实验设计与结果", roofline paragraph) places decoding on
 *     the memory-bandwidth roof and, with many candidates, on the compute
 *     roof; these two calls measure both roofs on the device itself, next to
 *     the kernels they bound.
 *  medusa_peak_hbm_read: reads `bytes` (rounded down to 16) of `buf` once,
 *     with 16-byte non-temporal loads; time it to get the read bandwidth.
 *     Use a buffer much larger than the 256 MB last-level cache.
 *  medusa_peak_mfma_bf16: `blocks` blocks of 4 waves, each wave running 4
 *     independent chains of `iters` v_mfma_f32_32x32x16_bf16 products on
 *     register operands (no memory traffic); medusa_peak_mfma_flops(blocks,
 *     iters) is the flop count of one call.
 *  sink: device, 16 bytes, 16-byte aligned; never written in practice (the
 *     results only decide a store, so the work cannot be elided).
 *  Errors: ERR_ARG (NULL, misaligned, empty), ERR_UNSUPPORTED, ERR_HIP. */
medusa_status medusa_peak_hbm_read(medusa_stream_t stream, const void *buf, size_t bytes, uint32_t *sink);
medusa_status medusa_peak_mfma_bf16(medusa_stream_t stream, int blocks, int iters, float *sink);
double medusa_peak_mfma_flops(int blocks, int iters);
/* The current device's compute units and its peak shader and memory clocks
 * (kHz, as the runtime reports them; 0 where not reported).  Host outputs,
 * each may be NULL.  ERR_HIP without a device. */
medusa_status medusa_device_info(int *compute_units, int *clock_khz, int *memory_clock_khz);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
