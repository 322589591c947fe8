/*
 * spec_verify.h — batched speculative-decoding verification on MI355X (gfx950).
 *
 * One call verifies B sequences.  For sequence b the caller passes the target
 * model's logits at K+1 positions and the drafter's logits at K positions,
 * plus the K drafted token ids.  The library
 *   1. applies temperature, then top-k, then top-p (on the renormalised top-k
 *      set) identically to every target and draft row, and normalises them to
 *      p_0..p_K and q_0..q_{K-1};
 *   2. accepts drafted token d_k while u_k * q_k(d_k) < p_k(d_k), i.e. with
 *      probability min(1, p/q), and stops at the first rejection j;
 *   3. emits d_0..d_{j-1} and then one more token: after a rejection a draw
 *      from max(0, p_j - q_j) normalised, or, when all K drafts are accepted,
 *      the bonus token drawn from p_K.
 * Greedy mode instead accepts the longest prefix with d_k == argmax p_k and
 * emits the target argmax at the first mismatch.
 *
 * Where these steps are defined:
 *  - accept test, stop at the first rejection, residual distribution and the
 *    identity that makes the output distribution equal to p: "FlashMap: Flow
 *    Map Speculative Decoding and the Mathematical Elimination of Suffix
 *    Decay", section 4 (The Rejection Sampling Invariant); "Speculative
 *    decoding and multi-token prediction: how LLMs generate faster", sections
 *    "Draft and verify" and "Why the output is identical";
 *  - K+1 target distributions, bonus token, greedy longest-prefix mode:
 *    "DFlash", section 4 (inference and distribution equivalence);
 *  - logits / temperature before the softmax: FlashMap page, section 5;
 *  - top-k and top-p applied the same way to both distributions:
 *    threatfrontier page, "Why the output is identical".
 *
 * Readings of points the pages leave open (all documented in the repository
 * design notes): accept on u * q < p with u in [0, 1) (so p = 0 is never
 * accepted and p >= q always is); top-k keeps every token whose logit is at
 * least the k-th largest (ties kept); top-p keeps a group of equal logits
 * while the mass of all strictly larger logits is below top_p (the top group
 * is always kept, the crossing group whole); when rounding leaves no
 * residual mass after a rejection the token is drawn from p_j; draws use
 * the inverse CDF in ascending token order.
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed low 32 bits, seed high 32 bits) and counter (b, k, purpose, 0);
 * purpose 0 = accept test at position k, uniform (w0 >> 8) * 2^-24;
 * purpose 1 = draw at stop position j, uniform
 * ((w0 >> 5) * 2^26 + (w1 >> 6)) * 2^-53.  A call is a pure function of its
 * inputs and seed: repeated calls give identical outputs.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  Inputs must
 *    stay alive and unmodified, and outputs untouched, until the stream has
 *    reached the end of the call.
 *  - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *    NULL means the null stream).  No call synchronises the device, except
 *    that the first call on a (device, stream) pair, or one that needs a larger
 *    workspace, allocates library-owned scratch memory (hipMalloc) and waits
 *    for the stream before releasing a smaller one.
 *  - Layouts are row-major and contiguous: target [B][K+1][V], draft
 *    [B][K][V], draft_tokens [B][K], out_tokens [B][K+1], out_num_accepted [B].
 *    Rows whose byte address is 16-byte aligned take the vector load path;
 *    other alignments are correct but slower.
 *  - Return values report host-checkable problems only (SPEC_E_*); device-side
 *    preconditions are documented and not checked: no NaN or +inf logits, and
 *    every row has at least one finite logit that survives its filters.
 *  - A drafted id outside [0, V) has p = q = 0 and is rejected.
 *  - out_tokens[b] holds d_0..d_{j-1}, then the emitted token, then -1 up to
 *    K+1 entries; out_num_accepted[b] = j in [0, K].
 *  - The library keeps one workspace per (device, stream): concurrent calls on
 *    the same stream from several host threads must be serialised by the
 *    caller; calls on different streams may overlap.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats of logits. */
typedef enum { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 } spec_dtype_t;

/* Status codes. */
typedef enum {
    SPEC_OK = 0,
    SPEC_E_INVALID = 1,     /* bad pointer, size, temperature, top_p, ... */
    SPEC_E_UNSUPPORTED = 2, /* unknown dtype code                         */
    SPEC_E_NOMEM = 3,       /* workspace allocation failed                */
    SPEC_E_LAUNCH = 4,      /* a HIP runtime call or kernel launch failed */
    SPEC_E_SCRATCH = 5      /* spec_verify_noalloc: the problem does not fit
                               the fixed scratch (SPEC_NOALLOC_SCRATCH_BYTES) */
} spec_status_t;

/* Per-row intermediates written by spec_verify_stats (32 bytes). */
typedef struct {
    float max_logit;       /* M: largest raw logit of the row (always kept)   */
    float thresh;          /* keep threshold: kept <=> x >= thresh (-inf: all) */
    int32_t n_kept;        /* number of kept tokens                           */
    int32_t flags;         /* SPEC_ROW_* bits                                 */
    double z_kept;         /* sum over kept tokens of exp((x - M) / T)        */
    double prob_at_token;  /* p_k(d_k) or q_k(d_k); 0 for an out-of-range id;
                              unused (NaN) for the bonus row p_K              */
} spec_row_stats_t;

#define SPEC_ROW_FILTERED 0x1  /* top-k or top-p active on this row          */
#define SPEC_ROW_EXACT_PATH 0x2 /* resolved by re-reading the row            */

/*
 * Sampling-mode verification (temperature > 0), or greedy semantics when
 * temperature == 0 (then draft_logits and draft_dtype are not used and may be
 * NULL / any value).
 *   target_logits  [B][K+1][V] in target_dtype
 *   draft_logits   [B][K][V]   in draft_dtype (may be NULL when K == 0)
 *   draft_tokens   [B][K] int32 (may be NULL when K == 0)
 *   B >= 0 (B == 0 is a no-op), K >= 0, V >= 1, B*(2K+1)*V < 2^40
 *   temperature    finite, >= 0
 *   top_k          <= 0 or >= V: disabled; otherwise keep logits >= the
 *                  top_k-th largest
 *   top_p          in (0, 1]; 1 disables it
 *   seed           key of the random stream
 *   out_tokens     [B][K+1] int32, out_num_accepted [B] int32
 *   stream         hipStream_t or NULL
 *   target_dtype, draft_dtype: spec_dtype_t codes
 * Returns SPEC_OK or an error code; on error nothing is launched.
 */
int spec_verify(const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, int B, int K, int V,
                float temperature, int top_k, float top_p, uint64_t seed,
                int32_t* out_tokens, int32_t* out_num_accepted, void* stream,
                int target_dtype, int draft_dtype);

/*
 * spec_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bitwise), kernels and errors as spec_verify, except
 * that it never allocates or frees: its scratch (row records, kept lists,
 * draw records and counters) lives in one fixed static device array of
 * SPEC_NOALLOC_SCRATCH_BYTES per GPU, which the GPU holds until the process
 * ends.  A problem whose scratch does not fit returns SPEC_E_SCRATCH before
 * any launch: with top-k / top-p each target row keeps an 80 KiB kept list,
 * so about B * (K+1) <= 400 target rows fit (the B = 32, K = 7 batch takes
 * 21 MB); unfiltered and greedy calls need a few hundred bytes per row and
 * per 1024 tokens of each sequence's stop row.  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (on different
 * streams or from different threads) race and must be serialised by the
 * caller.  What must start at zero is cleared by the call's first kernel.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, int B, int K, int V,
                        float temperature, int top_k, float top_p,
                        uint64_t seed, int32_t* out_tokens,
                        int32_t* out_num_accepted, void* stream,
                        int target_dtype, int draft_dtype);

/*
 * Per-sequence draft lengths (the serving engines' per-request number of
 * speculative tokens: "DFlash" page, section 2, on block size and
 * num_speculative_tokens) with per-position acceptance counters (the
 * measured acceptance by position in "FlashMap" section 6; threatfrontier,
 * "Practical guidance": measure the acceptance rate first).
 *   draft_lens     [B] int32 device array: sequence b verifies only its first
 *                  K_b = draft_lens[b] drafts (values are clamped to [0, K])
 *                  against target rows 0..K_b; the bonus token comes from row
 *                  K_b.  Rows past K_b are not read (the padded [B][K+1][V] /
 *                  [B][K][V] / [B][K] layout of spec_verify is kept).
 *   out_tokens     [B][K+1]: accepted drafts, the emitted token, then -1.
 *   pos_tested     [K] int32 or NULL: sequences whose accept test at position
 *                  k ran (k < K_b and num_accepted >= k).
 *   pos_accepted   [K] int32 or NULL: sequences that accepted position k.
 * Everything else as spec_verify (temperature == 0: greedy, accepting while
 * d_k equals the target argmax for k < K_b).  draft_lens must be non-NULL
 * when B > 0.  The counters are cleared by the call's first kernel and
 * counted with integer atomics by the kernels that write each sequence's
 * outputs, so they are exact and do not depend on order.
 */
int spec_verify_ragged(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_lens,
                       int B, int K, int V, float temperature, int top_k,
                       float top_p, uint64_t seed, int32_t* out_tokens,
                       int32_t* out_num_accepted, int32_t* pos_tested,
                       int32_t* pos_accepted, void* stream, int target_dtype,
                       int draft_dtype);

/*
 * Verification against point-mass drafts: a drafter that proposes each token
 * with certainty (a lookup table, n-gram or prompt-lookup proposer, or greedy
 * draft heads; "Speculative decoding and multi-token prediction: how LLMs
 * generate faster", sections "Draft and verify" and "Where drafts come
 * from") has q_k = delta(d_k), so no draft logits are read.  The test of
 * "Why the output is identical" (same page) then accepts d_k when
 * u_k < p_k(d_k); after the first rejection j the stop token is drawn from
 * p_j with d_j removed and renormalised; after K acceptances the bonus token
 * from p_K.  Temperature, top-k and top-p process the target rows as in
 * spec_verify (a point mass is unchanged by them).  Same arguments,
 * conventions, random stream and errors as spec_verify without draft_logits
 * and draft_dtype; temperature == 0 gives greedy semantics.  Reads only the
 * target logits: B*(K+1)*V*sizeof(target) bytes.
 */
int spec_verify_point(const void* target_logits, const int32_t* draft_tokens,
                      int B, int K, int V, float temperature, int top_k,
                      float top_p, uint64_t seed, int32_t* out_tokens,
                      int32_t* out_num_accepted, void* stream,
                      int target_dtype);

/*
 * Token-tree verification (multi-head / tree speculation: "Speculative
 * decoding and multi-token prediction: how LLMs generate faster", section
 * "Multi-head and tree speculation": the target evaluates all branches of a
 * proposal tree in one forward pass and the output follows one root path).  The pages leave the
 * rule for several candidates at one node open; the reading taken extends
 * the point-mass rule of spec_verify_point to siblings:
 *   node_tokens [B][N] int32 device array: token of node i.
 *   parents     [B][N] int32 device array: parent of node i, -1 for the root
 *               (the committed context) or a node index below i; any other
 *               value leaves node i unreachable.  N <= 1024.
 *   target_logits [B][N+1][V]: row 0 is the root's distribution, row i+1 the
 *               distribution after node i (the tree-attention pass).
 * From the root, the current node's children are tested in index order:
 * child c is accepted when u_c < p(x_c), where p is the current node's
 * processed row with the tokens of the siblings rejected before c removed
 * and renormalised (a repeated sibling token is therefore never accepted,
 * and a token outside [0, V) is always rejected).  An accepted child becomes
 * the current node.  When all children are rejected, the last token is drawn
 * from that remaining distribution (from the full row if nothing remains);
 * a leaf gives the bonus draw from its row.  u_c is the accept uniform of
 * counter (sequence, c); the draw uses the sample uniform of counter
 * (sequence, r), r the row of the node where the walk stopped; so a tree
 * that is one chain reproduces spec_verify_point.  temperature == 0: follow
 * the first child whose token is the row's argmax (lowest index among equal
 * maxima), then emit that argmax.
 * Outputs (device arrays): out_tokens [B][N+1] (the path's tokens, the last
 * token, then -1); out_num_accepted [B] (path length); out_path [B][N] (node
 * indices of the path, then -1; may be NULL).  Temperature, top-k, top-p,
 * seed, stream, dtype and error codes as spec_verify.  Reads the target
 * logits once: B*(N+1)*V*sizeof(target) bytes.
 */
int spec_verify_tree(const void* target_logits, const int32_t* node_tokens,
                     const int32_t* parents, int B, int N, int V,
                     float temperature, int top_k, float top_p, uint64_t seed,
                     int32_t* out_tokens, int32_t* out_num_accepted,
                     int32_t* out_path, void* stream, int target_dtype);

/*
 * Greedy verification straight from the target's last hidden states, the
 * unembedding product fused in ("FlashMap: Flow Map Speculative Decoding and
 * the Mathematical Elimination of Suffix Decay", section 3: a position's
 * logits are its hidden state times the transposed unembedding matrix; the
 * greedy rule of "DFlash", section 4, as spec_verify_greedy):
 *   hidden     [B][K+1][H] bf16 device array: the target's final hidden state
 *              at each verified position (16-byte aligned);
 *   w_unembed  [V][H] bf16 device array: the unembedding (LM head) matrix
 *              (16-byte aligned);
 *   H          hidden size, a multiple of 8.
 * The logits hidden . w_unembed^T are computed in tiles on the matrix cores
 * (bf16 products, fp32 accumulation) and reduced to each row's argmax
 * (lowest index among equal maxima) without being written to memory; the
 * accepted prefix and the emitted token are as spec_verify_greedy.  Logits
 * whose top two values lie within the fp32 accumulation error of each other
 * may resolve to either.  Outputs, stream and error codes as spec_verify.
 */
int spec_verify_greedy_hidden(const void* hidden, const void* w_unembed,
                              const int32_t* draft_tokens, int B, int K, int V,
                              int H, int32_t* out_tokens,
                              int32_t* out_num_accepted, void* stream);

/*
 * The unembedding product: a position's logits are its hidden state times
 * the transposed unembedding (LM head) matrix ("FlashMap: Flow Map
 * Speculative Decoding and the Mathematical Elimination of Suffix Decay",
 * section 3).
 *   hidden      [R][H] bf16 device array (16-byte aligned)
 *   w_unembed   [V][H] bf16 device array (16-byte aligned); H a multiple of 8
 *   out_logits  [R][V] bf16 device array: each logit is the product formed
 *               with bf16 products accumulated in fp32 on the matrix cores,
 *               rounded to bf16 (nearest, ties to even), as a bf16 LM head
 *               outputs its logits.  Exact whenever the fp32 sums are (for
 *               instance with small-integer inputs); otherwise each logit is
 *               the bf16 rounding of a value within the fp32 accumulation
 *               error (at most H * 2^-24 * sum |h w|) of the exact product.
 * R == 0 is a no-op.  Stream and error codes as spec_verify.
 */
int spec_lm_head_logits(const void* hidden, const void* w_unembed, int R,
                        int V, int H, void* out_logits, void* stream);

/*
 * Verification from hidden states with the unembedding shared by target and
 * drafter (FlashMap page, section 5: the drafter's logits come from the
 * target's LM head; "DFlash" section 5: the drafter shares the target's
 * token embedding and LM head):
 *   target_hidden [B][K+1][H] bf16: the target's final hidden state at each
 *                 verified position;
 *   draft_hidden  [B][K][H] bf16: the drafter's output state at each drafted
 *                 position (may be NULL when K == 0);
 *   w_unembed     [V][H] bf16, the shared unembedding matrix.
 * The logits of all B(2K+1) rows come from one pass over w_unembed as in
 * spec_lm_head_logits (bf16), and are then verified exactly as spec_verify
 * verifies bf16 target and draft logits (temperature, top-k, top-p, seed,
 * outputs and errors as there; temperature == 0 runs
 * spec_verify_greedy_hidden on the target rows).  The logits stay in a
 * library-owned buffer per (device, stream), B(2K+1)*V*2 bytes, written once
 * and read once: exact top-p needs every logit of a row (or a second pass
 * over w_unembed, which is larger at these sizes).
 */
int spec_verify_hidden(const void* target_hidden, const void* draft_hidden,
                       const void* w_unembed, const int32_t* draft_tokens,
                       int B, int K, int V, int H, float temperature,
                       int top_k, float top_p, uint64_t seed,
                       int32_t* out_tokens, int32_t* out_num_accepted,
                       void* stream);

/*
 * Greedy verification: g_k = argmax of target row k (lowest index among equal
 * maxima), accept while d_k == g_k, emit g_j at the first mismatch j (or the
 * bonus argmax g_K).  Reads target logits only.  Same conventions as
 * spec_verify ("DFlash", section 4: the longest prefix matching the target's
 * greedy choices).
 */
int spec_verify_greedy(const void* target_logits, const int32_t* draft_tokens,
                       int B, int K, int V, int32_t* out_tokens,
                       int32_t* out_num_accepted, void* stream,
                       int target_dtype);

/*
 * spec_verify plus the per-row intermediates: target_stats [B][K+1] and
 * draft_stats [B][K] (device arrays of spec_row_stats_t, either may be NULL).
 * Sampling mode only (temperature > 0).  Outputs are identical to
 * spec_verify's for the same arguments.
 */
int spec_verify_stats(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, int B, int K, int V,
                      float temperature, int top_k, float top_p, uint64_t seed,
                      int32_t* out_tokens, int32_t* out_num_accepted,
                      void* stream, int target_dtype, int draft_dtype,
                      spec_row_stats_t* target_stats,
                      spec_row_stats_t* draft_stats);

/*
 * Diagnostic: the uniforms the verifier draws for `seed`, computed by the
 * same device generator: u_accept [B][K] (purpose 0) and u_sample [B][K+1]
 * (purpose 1), as doubles in device memory.  Either pointer may be NULL.
 */
int spec_rng_uniforms(uint64_t seed, int B, int K, double* u_accept,
                      double* u_sample, void* stream);

/*
 * Measurement hook: when both are non-NULL hipEvent_t handles, the next
 * verification call on logits (sampling or greedy) records `before` on its
 * stream just before launching its streaming (dominant) kernel and `after`
 * just after it (for greedy calls below 512 sequences that kernel also
 * writes the outputs); the hook is then cleared.  Passing NULLs clears it.
 * Not thread-safe with concurrent calls.
 */
int spec_profile_events(void* before, void* after);

/* Human-readable text for a status code (static storage). */
const char* spec_status_string(int status);

/* Free every workspace the library holds (waits for their streams). */
void spec_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
