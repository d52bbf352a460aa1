/*
 * specverify.h -- C ABI of the MI355X (gfx950) speculative-decoding
 * verify-and-accept library, libspecverify.so.
 *
 * Pages the operations follow (cited by title and section):
 *   [PT] "Decodificacao Especulativa e EAGLE-3", ai-engineering.academy,
 *        Fase 10 - Licao 15 (the same lesson exists in Persian on
 *        nextadmin.net).
 *   [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异", caijizhuo.github.io.
 * Notation: q = verifier (target) distribution, p = draft distribution.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or synchronises.  All work is enqueued
 *     on `stream` (a hipStream_t; 0 = the null stream) in order, so outputs
 *     are ready when that stream reaches the point after the call.
 *   - Host-checkable argument errors return a status before anything is
 *     launched (SV_EINVAL, SV_EDTYPE, SV_ESHAPE, SV_EALIGN, SV_EWORKSPACE);
 *     SV_EHIP reports a failed launch.  Outputs are then unspecified.
 *   - Data errors found on the device are reported per sequence, never by
 *     status: out_num_accepted[b] = -1 and out_tokens row b all -1.  They are
 *     NaN or +inf in a logit row the outcome reads, a row that is all -inf, a
 *     token outside [0, V), a parent outside [0, n), or a walk longer than
 *     max_depth.
 *   - Blocks of one launch hand data to later blocks of the same launch
 *     through records (a block waits only for blocks dispatched before it).
 *     Every such wait is bounded (2^19 polls); one that runs out fails its
 *     sequence with out_num_accepted[b] = -2 (token row all -1).  That is
 *     never expected and is not a property of the data.  For tests of this
 *     path the bound is read from the environment variable
 *     SV_TEST_SPIN_LIMIT (polls, 0 ... 2^19) at each call when it is set.
 *   - Logit rows: element (b, r, t) of a logits array lives at
 *     base + (b*seq_stride + r*row_stride + t) elements.  The base must be
 *     aligned to the element size (SV_EALIGN otherwise); V and the strides
 *     are arbitrary.  Rows whose start is 16-byte aligned (e.g. V a multiple
 *     of 8 for bf16, of 4 for fp32) stream entirely as 16-byte vectors;
 *     others take a short scalar head.
 *   - Temperature T > 0 divides both q- and p-logits before the softmax.
 *   - Uniforms: Philox4x32-10 (Salmon et al., SC'11), key = seed, counter =
 *     (position, sequence, round low 32 bits, (round bits 32..59) << 4).  The
 *     accept uniform of position/node n is the 53-bit double of words 0,1 of
 *     the block at position n; the sampling uniform of slot s is the one of
 *     words 2,3 of the block at position s.  A call is a pure function of its
 *     inputs and (seed, round).
 *   - Workspace (verify calls): caller-owned device memory, ZERO-FILLED once
 *     before its first use.  Each call tags its records and counters with
 *     its own number (the low word of a 64-bit call counter that starts at a
 *     value drawn when the library is loaded), so after that single zero
 *     fill a workspace is reused as is by any later call (chain or tree, any
 *     sizes that fit).  A record or counter left by an earlier call is
 *     recognised as stale unless its call's number matches this one's in the
 *     low 32 bits.
 *   - Reentrant; calls on different streams may overlap as long as they use
 *     different workspaces and outputs.  The only process-wide state is that
 *     call counter (an atomic), cached occupancy figures and the scratch
 *     array of spec_verify_chain_noalloc.
 *   - A chain verify call is one kernel launch (for bf16 logits the value
 *     table, then row statistics, accept tests, chunk sums and final step in
 *     one grid); chains of bf16 logits whose rows are not 16-byte aligned
 *     take two (row statistics and accept tests; chunk sums and final step);
 *     a tree verify call takes two (row statistics, the table, accept tests
 *     and walk; sampling).  Row statistics are
 *     summed per fixed segment of about 64K tokens and combined in segment
 *     order, so results do not depend on the device's compute-unit count.
  */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sv_status {
    SV_OK = 0,
    SV_EINVAL = 1,      /* NULL required pointer, bad count, T <= 0, ... */
    SV_EDTYPE = 2,      /* dtype not SV_F32 / SV_BF16 */
    SV_ESHAPE = 3,      /* N > 64, T+1 > 1024, max_depth < 0, ... */
    SV_EALIGN = 4,      /* logits not element-aligned / KV rows not 16-byte aligned */
    SV_EWORKSPACE = 5,  /* workspace NULL or smaller than required */
    SV_EHIP = 6,        /* a HIP launch failed */
    SV_ESCRATCH = 7     /* sizes beyond spec_verify_chain_noalloc's static scratch */
};

enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 };

/* Tree walks (spec_verify_tree's `walk`). */
enum sv_walk {
    SV_WALK_FIRST_ACCEPTED = 0, /* descend into the lowest-index accepted child */
    SV_WALK_BEST_CHILD = 1      /* the pages' literal walk: only the lowest-index
                                   child is tried; its rejection ends the walk */
};

/* Optional timing hook: when non-NULL, each non-NULL event is stamped by a
 * kernel of the call on `stream`: `begin` by the start of the row kernel
 * (the call's first kernel), `rows_done` by that kernel's end, and `end` by
 * the end of the call's last kernel.  A caller can time the call, and its
 * row-statistics kernel alone, without events between the kernels. */
typedef struct sv_timing {
    hipEvent_t begin;
    hipEvent_t rows_done;
    hipEvent_t end;
} sv_timing;

/* ABI version (incremented on any change of a signature or of an output convention). */
int sv_abi_version(void);

/* Static text for a status code. */
const char* sv_status_string(int status);

/* Workspace bytes spec_verify_chain needs for (B, N, V); 0 on bad sizes. */
size_t sv_chain_workspace_bytes(int B, int N, int V);

/* Workspace bytes spec_verify_tree needs for (B, T, V); 0 on bad sizes. */
size_t sv_tree_workspace_bytes(int B, int T, int V);

/*
 * spec_verify_chain -- one verify round of B independent chains of N draft
 * tokens ([PT] "O Conceito": N stacked accept calls over one verifier pass
 * that returns q_1..q_{N+1}; walk left to right; at the first rejection j
 * sample residual(q_j, p_j) and stop; if all are accepted sample a bonus
 * token from q_{N+1}.  [PT] Implementando, Passo 1 (accept iff
 * u < min(1, q(d)/p(d)), zero draft probability accepts) and Passo 2 (the
 * residual (q-p)_+ normalised, q itself when it sums to zero).  [ZH]
 * section 2 states the same three steps.)
 *
 *   target_logits  [B, N+1, V]  q-logits; row i tests draft d_{i+1}, row N is
 *                               the bonus distribution (read only when all N
 *                               drafts are accepted).
 *   draft_logits   [B, N, V]    p-logits (may be NULL when N == 0).
 *   dtype          SV_F32 or SV_BF16 (both logit arrays).
 *   draft_tokens   [B, N] int32 d_1..d_N.
 *   B >= 0, 0 <= N <= 64, V >= 1, T > 0.
 * Outputs (out_tokens and out_num_accepted required, the rest optional):
 *   out_tokens        [B, N+1] int32: d_1..d_k, the correction or bonus
 *                     token, then -1.
 *   out_num_accepted  [B] int32: k in [0, N], -1 on a data error, -2 if a
 *                     wait timed out (see the conventions).
 *   out_accept        [B, N] int8: the accept decision of every position
 *                     (positions after the first rejection are decided too).
 *   out_probs         [B, N, 2] float: (q_i(d_i), p_i(d_i)).
 *   out_residual_mass [B] double: sum_t (q_{k+1}(t) - p_{k+1}(t))_+ after a
 *                     rejection, 0 after the bonus.
 * KV rows ([PT] Implementando, Passo 4: after the round the KV cache keeps
 * the pending token and the k accepted drafts), optional: kv_len_in [B]
 * int32 is L0, the KV row of the pending token (position 0); the verify
 * pass wrote position i at row L0 + i.  out_src_rows [B, N+1] int32 gets
 * L0 + i for i <= k and -1 after; out_kv_len [B] int32 gets L0 + k + 1.  A
 * failed sequence gets -1 rows and keeps L0.  kv_len_in is required when
 * either output is given (SV_EINVAL otherwise); these are the values
 * kv_compact_indices(NULL, ...) computes, without its launch.
 * Sampling is an inverse CDF in token-id order: the first token whose
 * running weight exceeds u*W, W the total weight, accumulated in double.
 * workspace: device memory of at least sv_chain_workspace_bytes(B, N, V)
 * bytes, 16-byte aligned, zero-filled before its first use (see the
 * conventions above).
 */
int spec_verify_chain(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                      const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                      const int32_t* draft_tokens, int B, int N, int V, uint64_t seed, uint64_t round,
                      float temperature, int32_t* out_tokens, int32_t* out_num_accepted, int8_t* out_accept,
                      float* out_probs, double* out_residual_mass, const int32_t* kv_len_in, int32_t* out_src_rows,
                      int32_t* out_kv_len, void* workspace, size_t workspace_bytes, const sv_timing* timing,
                      hipStream_t stream);

/*
 * spec_verify_chain_noalloc -- spec_verify_chain without a workspace
 * argument, for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * outputs are those of spec_verify_chain.  The call allocates nothing: its
 * workspace is a static device array of the library,
 * SV_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, zero when the library is loaded
 * and kept until the process ends (chains of B=256 N=7 V=128256
 * need about 1.3 MB).  Sizes whose sv_chain_workspace_bytes exceed it
 * return SV_ESCRATCH before any HIP call.  Every call on one GPU shares that
 * GPU's array (each call tags its records, so what an earlier call left
 * needs no clearing); calls that overlap in time on one GPU race and must
 * not be made.  The first call on a device looks the array's address up
 * with hipGetSymbolAddress (with that device current); SV_EHIP if that
 * fails.
 */
#define SV_NOALLOC_SCRATCH_BYTES (4u << 20)
int spec_verify_chain_noalloc(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                              const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                              const int32_t* draft_tokens, int B, int N, int V, uint64_t seed, uint64_t round,
                              float temperature, int32_t* out_tokens, int32_t* out_num_accepted,
                              int8_t* out_accept, float* out_probs, double* out_residual_mass,
                              const int32_t* kv_len_in, int32_t* out_src_rows, int32_t* out_kv_len,
                              const sv_timing* timing, hipStream_t stream);

/*
 * spec_verify_tree -- one verify round over B flattened draft trees ([ZH]
 * section 3: the tree is flattened into a sequence with numbered nodes and
 * verified by one pass in which a node sees only itself and its ancestors;
 * section 4, "eagle_round" step 4: walk from the root accepting children;
 * [PT] O Conceito, EAGLE-2: the verifier scores every candidate in one pass
 * and the most probable accepted path is kept).
 *
 * Reading of the walk: node n >= 1 is tested with q and p at parent(n) and
 * its accept uniform; from the root, the walk descends into the
 * lowest-index accepted child (siblings are expected in descending draft
 * probability, so this is the most probable accepted path); it stops at a
 * leaf (bonus sampled from that leaf's q) or at a node none of whose
 * children is accepted (residual of that node's q and p).  The sampling
 * uniform is that of slot depth(stop) + 1, so a path-shaped tree reproduces
 * spec_verify_chain bit for bit.
 *
 * walk = SV_WALK_BEST_CHILD follows the pages' pseudocode literally ([ZH]
 * section 4, "eagle_round" step 4: take the node's best child; accept and
 * go on, or reject, resample and end): from each node only its
 * lowest-index child is tried, and its rejection stops the walk with the
 * residual at that node even when a sibling was accepted.  This is the
 * chain verify of the tree's best-child path.  Every node is still tested
 * (out_accept, out_probs).
 *
 *   target_logits  [B, T+1, V]  q-logits per node (node 0 = root).
 *   draft_logits   [B, T+1, V]  p-logits per node (rows of leaves unread).
 *   node_tokens    [B, T+1] int32 (entry 0 unread).
 *   parents        [T+1] int32 when parents_shared != 0, else [B, T+1];
 *                  parents[n] in [0, n) for n >= 1 (entry 0 unread).
 *   0 <= T <= 1023, 0 <= max_depth <= T; a walk longer than max_depth is a
 *   data error, so max_depth should be at least the tree's depth.
 *   walk: SV_WALK_FIRST_ACCEPTED or SV_WALK_BEST_CHILD (else SV_EINVAL).
 * Outputs (tokens, path_nodes, num_accepted required):
 *   out_tokens        [B, max_depth+1] int32: tokens of the accepted path,
 *                     then the correction/bonus token, then -1.
 *   out_path_nodes    [B, max_depth+1] int32: 0, the accepted nodes, -1.
 *   out_num_accepted  [B] int32: accepted depth k, -1 on a data error, -2 if
 *                     a wait timed out.
 *   out_accept        [B, T+1] int8: the decision of every node (node 0: 1).
 *   out_probs         [B, T+1, 2] float: (q_par(tok_n), p_par(tok_n)), node 0
 *                     (0, 0).
 *   out_residual_mass [B] double, as for chains.
 * KV rows, optional, as for chains with the path: node n was written at row
 * L0 + n, so out_src_rows [B, max_depth+1] gets L0 + path_nodes[i] for
 * i <= k ([ZH] section 3: the accepted path's rows are kept and moved
 * together) and out_kv_len L0 + k + 1; the in-place gather of the KV rows
 * themselves is kv_compact_indices.
 * workspace: at least sv_tree_workspace_bytes(B, T, V) bytes, zero-filled
 * before first use, as for chains.
 */
int spec_verify_tree(const void* target_logits, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                     const void* draft_logits, int64_t drf_seq_stride, int64_t drf_row_stride, int dtype,
                     const int32_t* node_tokens, const int32_t* parents, int parents_shared, int B, int T, int V,
                     int max_depth, int walk, uint64_t seed, uint64_t round, float temperature,
                     int32_t* out_tokens, int32_t* out_path_nodes, int32_t* out_num_accepted, int8_t* out_accept,
                     float* out_probs, double* out_residual_mass, const int32_t* kv_len_in, int32_t* out_src_rows,
                     int32_t* out_kv_len, void* workspace, size_t workspace_bytes, const sv_timing* timing,
                     hipStream_t stream);

/*
 * kv_compact_indices -- KV rollback and compaction after a verify round
 * ([PT] Implementando, Passo 4 and "Reversao de KV cache": a logical KV
 * length truncated at the rejection; [ZH] section 3: after acceptance the
 * KV rows of the accepted path are copied together and the other branches
 * dropped).
 *
 * kv_len_in[b] = L0 is the KV row of node 0 (the pending token); the verify
 * pass wrote node n (chain position n) at row L0 + n.  Accepting k drafts
 * keeps k + 1 rows: out_src_rows[b, i] = L0 + path[i] for i <= k (path =
 * identity for chains, path_nodes == NULL), -1 after; out_kv_len[b] =
 * L0 + k + 1.  A sequence with num_accepted < 0 keeps out_kv_len = L0 and
 * gets -1 rows.  A path that is not strictly increasing from node 0, or rows
 * outside [0, kv_rows), mark the sequence with out_kv_len = -1 and leave its
 * KV untouched.
 *
 * When kv != NULL the gather is done in place: for every plane (K and V of
 * every layer, plane_stride bytes apart), row L0 + path[i] of sequence b
 * (seq_stride bytes per sequence, row_stride bytes per row, row_bytes bytes
 * copied) moves to row L0 + i.  Every source row is read before it can be
 * overwritten.  kv, the strides and row_bytes must be multiples of 16.
 */
int kv_compact_indices(const int32_t* path_nodes, const int32_t* num_accepted, const int32_t* kv_len_in, int B,
                       int max_depth, int32_t* out_src_rows, int32_t* out_kv_len, void* kv, int kv_rows,
                       int64_t seq_stride, int64_t row_stride, int row_bytes, int n_planes, int64_t plane_stride,
                       hipStream_t stream);

/*
 * tree_attention_mask -- the verifier-side inputs of a tree verify pass
 * ([ZH] section 3, "草稿树与树形注意力掩码": the draft tree is flattened into
 * one sequence of numbered nodes and every node attends only to itself and
 * its ancestors, never to its siblings, so one verifier forward pass scores
 * every node; [PT] "Reversao de KV cache": the verifier runs attention with a
 * non-causal mask that follows the tree's topology).
 *
 * parents as for spec_verify_tree: [T+1] shared by every sequence
 * (parents_shared != 0) or [B, T+1]; parent[0] = -1 and 0 <= parent[n] < n.
 * For node n of sequence b:
 *   out_mask [B, T+1, W] uint64, W = ceil((T+1)/64): bit (j & 63) of word
 *     (j >> 6) of row n is set iff node j is n or an ancestor of n (the tree
 *     part of the attention mask; every node also sees the KV prefix, which
 *     the mask does not cover).
 *   out_positions [B, T+1] int32: L0 + depth(n), with depth(0) = 0 and
 *     L0 = kv_len_in[b] (the KV row of node 0, as for kv_compact_indices;
 *     0 when kv_len_in is NULL): node n's position id.
 * A sequence whose parents break the rule gets an all-zero mask and -1
 * positions.  0 <= T <= 1023; out_mask and out_positions are required.
 */
int tree_attention_mask(const int32_t* parents, int parents_shared, const int32_t* kv_len_in, int B, int T,
                        uint64_t* out_mask, int32_t* out_positions, hipStream_t stream);

/*
 * EAGLE-2 dynamic draft tree, built level by level on the device ([ZH]
 * section 4, "eagle_round" step 2: every frontier node adds its top-k draft
 * tokens as children whose score is the parent's score times p(token), and
 * the best nodes are picked to grow next; section 5, EAGLE-2: nodes are
 * allotted globally by that score, and the tree keeps the `budget` best).
 * The draft model runs between the levels (not here): the caller feeds
 * each level's frontier rows to tree_expand, picks the next frontier with
 * tree_select, and flattens the tree with tree_finalize.
 *
 * Candidate table (caller-owned device arrays, n_max <= 2048 entries per
 * sequence, entry (b, i) at b*n_max + i): cand_token, cand_parent (the
 * parent's candidate id; -1 = the root), cand_level (1 = child of the
 * root), cand_score (double: the sum of ln p along the path, i.e. the
 * logarithm of the pages' product of probabilities; NaN marks a failed row).
 * Creation order is the candidate id; ties in score go to the lower id.
 */

/*
 * tree_expand -- one level: frontier row f of sequence b (logits at
 * frontier_logits + (b*seq_stride + f*row_stride) elements, V of them,
 * dtype SV_F32 / SV_BF16) gives its top-k tokens by (logit desc, token asc)
 * with p = softmax(logits / temperature), as candidates offset + f*topk + r
 * (r = rank): token, parent frontier_ids[b*F + f] (NULL: -1, the root),
 * level, score frontier_score[b*F + f] (NULL: 0) + ln p(token).  The row's
 * log-sum-exp sums fp32 exp2 terms in double (about 1e-8 relative).  A row
 * with NaN or +inf, or of -inf only, gives NaN scores.  1 <= topk <= 16,
 * topk <= V, offset + F*topk <= n_max <= 2048.
 */
int tree_expand(const void* frontier_logits, int64_t seq_stride, int64_t row_stride, int dtype, int B, int F, int V,
                int topk, float temperature, const int32_t* frontier_ids, const double* frontier_score, int level,
                int n_max, int offset, int32_t* cand_token, int32_t* cand_parent, int32_t* cand_level,
                double* cand_score, hipStream_t stream);

/*
 * tree_select -- the next frontier: of candidates [offset, offset + count)
 * of each sequence, the k best by (score desc, id asc), in that order:
 * out_ids [B, k] (candidate ids) and out_score [B, k].  NaN ranks lowest.
 */
int tree_select(const double* cand_score, int B, int n_max, int offset, int count, int k, int32_t* out_ids,
                double* out_score, hipStream_t stream);

/*
 * tree_finalize -- the kept set, the `budget` best of candidates [0, n) by
 * (score desc, id asc) (ancestor-closed: a child never outscores its parent
 * and is created after it), numbered 1..budget by (level asc, score desc,
 * id asc): out_parents, out_tokens, out_depth [B, budget+1] int32 and
 * out_score [B, budget+1] double; node 0 is the root (parent -1, token 0,
 * depth 0, score 0).  out_parents feeds spec_verify_tree and
 * tree_attention_mask.  A sequence with a NaN score gets -1 (score 0) in
 * every slot.  1 <= budget <= n <= n_max <= 2048.
 */
int tree_finalize(const int32_t* cand_token, const int32_t* cand_parent, const int32_t* cand_level,
                  const double* cand_score, int B, int n_max, int n, int budget, int32_t* out_parents,
                  int32_t* out_tokens, int32_t* out_depth, double* out_score, hipStream_t stream);

/*
 * sv_sample_draft -- draft tokens d ~ softmax(z / T) ([PT] O Conceito and
 * Implementando, Passo 1: the draft proposes d ~ p; [ZH] section 2: each
 * draft token is drawn from the draft model's softmax).  Row r of sequence
 * b, at logits + (b*seq_stride + r*row_stride) elements (V of them, dtype
 * SV_F32 / SV_BF16), gives out_tokens[b*R + r] by the verify step's inverse
 * CDF in token order (the first token whose running weight exceeds u*W, W
 * the total; the last token of positive weight if rounding leaves none;
 * double weights: for bf16 rows exp(z/T) from a per-block table over the
 * bf16 grid (one rounding each), otherwise, and for rows with a logit above
 * 700 T or a total below 1e-280, exp((z - ref)/T) by a table-driven fp64
 * exp (~1e-11 relative) against a running reference; accumulated in
 * double, so the draw is the inverse CDF of softmax(z/T) to ~1e-11 and ln
 * p within ~1e-11) with the uniform of
 * Philox stream 1: key seed, counter (pos0 + r, b, round low word,
 * (round high word << 4) | 1), words 0 and 1 as a 53-bit double, so draft
 * draws never reuse a verify uniform.  out_logprob[b*R + r] (may be NULL):
 * ln p(token) in double.  A row with NaN or +inf, or only -inf, gives -1
 * and NaN.  1 <= V <= 524288, pos0 >= 0, pos0 + R < 2^32.  One launch (a
 * block per row), no workspace.
 */
int sv_sample_draft(const void* logits, int64_t seq_stride, int64_t row_stride, int dtype, int B, int R, int V,
                    float temperature, uint64_t seed, uint64_t round, int pos0, int32_t* out_tokens,
                    double* out_logprob, hipStream_t stream);

/*
 * sv_philox_uniforms -- the uniforms the verify step draws, for tests of
 * the device generator: for sequences [0, nseq) and positions 1..npos,
 * out_acc[s*npos + p-1] and out_samp[s*npos + p-1] (device double arrays,
 * either may be NULL).
 */
int sv_philox_uniforms(uint64_t seed, uint64_t round, int nseq, int npos, double* out_acc, double* out_samp,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
