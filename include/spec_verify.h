/*
 * spec_verify.h -- batched verification of drafted tokens on AMD MI355X (gfx950).
 *
 * Speculative decoding lets a small draft model propose a run of tokens that
 * the large target model then checks in one parallel pass (MineDraft page,
 * section 1; SpecTr-GBV page, section 1).  This library implements that check
 * for a batch of B requests, each with K i.i.d. drafted blocks of length L
 * over a vocabulary of V tokens, given the target and draft logits:
 *
 *   spec_verify_token       token-level speculative sampling (K = 1): accept
 *                           token x with probability min(1, p(x)/q(x)), stop at
 *                           the first rejection and resample from the residual
 *                           norm(max(p - q, 0)) -- the standard rule the
 *                           speculative-decoding pages build on;
 *   spec_verify_block       greedy block verification, GBV (K = 1): the whole
 *                           block is verified jointly, the single-draft method
 *                           of the SpecTr-GBV page, section 1;
 *   spec_verify_multidraft  GBV over K i.i.d. drafts as the SpecTr-GBV page,
 *                           section 2 ("algorithmic procedure", steps 1-5),
 *                           describes it: walk the drafts, skip rejected
 *                           sub-blocks, keep the longest accepted prefix tau,
 *                           draw the correction from the target (tau = L) or
 *                           from the residual (tau < L), one O(V) sweep per
 *                           selection step and no search over a scaling factor
 *                           (section 3, efficiency);
 *   spec_verify_spectr      SpecTr, the multi-draft baseline the SpecTr-GBV page
 *                           compares against (sections 1 and 3): the K drafts are
 *                           verified position by position, each selection step
 *                           searching a scaling factor rho (k-sequential
 *                           selection; the rule is stated below).
 *
 * Every call is asynchronous on the caller's HIP stream: it validates its
 * arguments on the host, launches kernels and returns without synchronising.
 * The library never allocates device memory; scratch comes from the caller's
 * workspace (spec_verify_multidraft_noalloc uses scratch the library holds
 * itself).  Calls that share a workspace must be ordered on one stream.
 *
 * Work done per request: the softmax statistics of the rows the walk reads
 * first (the root pair and the rows of each draft with a new first token) are
 * streamed once from HBM; the walk then runs, and for K > 1 a draft that
 * continues below an accepted node makes a second round stream the rows
 * below that node for every draft sharing it.  Rows that the rules never
 * read are never loaded.
 *
 * Notation.  T_b is request b's temperature; the temperature softmax of a logit
 * row l is pi(v) = exp(l_v / T_b) / sum_v' exp(l_v' / T_b).  For draft k of
 * request b, target row j (j = 0..L) and draft row j (j = 0..L-1) are the
 * target and draft distributions of the token at position j+1, given the
 * prefix X[b][k][0..j-1]; X[b][k][j] was drawn from draft row j.
 *
 * Node rows.  Drafts of one request that share the prefix X[..][0..j-1] stand at
 * the same node of the draft tree, so their rows j must describe the same
 * distribution.  The library reads each node's rows from the lowest-index draft
 * with that prefix and never reads the duplicates, so a caller may leave them
 * unwritten.  (The pages do not fix this; it is the reading that keeps every
 * draft at a node tested against one distribution.)
 *
 * Decision rules, stated precisely:
 *  - tests are strict: a test with acceptance probability h accepts iff u < h,
 *    with u in [0, 1) taken from u_accept[b][k][m-1] for position m of draft k;
 *  - among several accepted positions of one block the largest wins;
 *  - the correction is the inverse-CDF draw in token-id order:
 *    y = min{v : C_v > u_correct[b] * Z}, C_v = sum_{v' <= v} omega(v'),
 *    Z = C_{V-1}, over the (unnormalised) correction weights omega;
 *  - the K-draft residual at a node s is omega(v) = [v not in H] *
 *    max(alpha p_s(v) - beta q_s(v), 0); a rejection adds the residual mass N
 *    to beta; a draft whose token at s is already in H is rejected without a
 *    test (its uniforms are not consumed) and still adds N to beta;
 *  - SpecTr at position j (node s = the accepted prefix, n = the number of drafts
 *    on it): beta(rho) = sum_v min(q_s, p_s/rho), c = sum_{i<n} (1 - beta)^i,
 *    rho* = the smallest rho in [1, n] with c <= rho (rho* = 1, c = 1 for n = 1);
 *    the drafts on the prefix are tested in index order with
 *    h = min(1, p_s(x)/(rho* q_s(x))) and u = u_accept[b][k][j]; the first
 *    success extends the prefix (draft_index = that draft), no success ends the
 *    walk with tau = j and a correction from max(p_s - c min(q_s, p_s/rho*), 0).
 *    rho* is found to about 1e-7 relative (fp32 evaluation of the rows).
 * Every probability is formed from fp32 exponentials with fp64 sums; a request
 * with a decision within the fp32 error of its threshold is taken again in fp64
 * (SV_FLAG_REDONE), so integer outputs match exact arithmetic except where a
 * decision lies within fp64 rounding of its threshold.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Nothing is launched when a call returns anything but SV_OK. */
typedef enum {
    SV_OK = 0,
    SV_EINVAL = 1,        /* null pointer, size out of range, K != 1 for token/block */
    SV_EUNSUPPORTED = 2,  /* dtype or size this build does not handle */
    SV_EHIP = 3,          /* a HIP runtime call failed (no device, launch error) */
    SV_EWORKSPACE = 4     /* workspace missing, misaligned or too small */
} sv_status;

/* Element type of both logit tensors. */
typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Limits of this build. */
#define SV_MAX_K 64
#define SV_MAX_L 16
#define SV_MAX_V (1 << 22)

/* Per-request flag bits (sv_outputs.flags). */
#define SV_FLAG_DEGENERATE 1  /* a residual of zero mass was met (rounding only);
                                 the node's target distribution was used instead */
#define SV_FLAG_INVALID 2     /* request data the rules cannot act on: T not a
                                 positive finite number, a token outside [0, V),
                                 a uniform outside [0, 1), or a node row that the
                                 rules read and that is not a distribution (NaN,
                                 +inf, all -inf) */
#define SV_FLAG_NEAR_TIE 4    /* a decision came within SV_NEAR_TIE of its
                                 threshold: an acceptance test with |u - h| <
                                 SV_NEAR_TIE, or the correction draw with u Z
                                 within SV_NEAR_TIE Z of a boundary of the
                                 cumulative weights.  The exponentials are fp32,
                                 so such a decision may differ from one taken in
                                 exact arithmetic; every other decision cannot */
#define SV_NEAR_TIE 1e-5
#define SV_FLAG_REDONE 8      /* the request was taken again in fp64 because one of
                                 its decisions came within SV_NEAR_TIE, or within a
                                 first-order estimate of the fp32 error (GBV tests
                                 whose h = R / (R + 1 - w) is ill-conditioned), of
                                 its threshold; its outputs, SV_FLAG_NEAR_TIE (from
                                 the fp64 margins), accept_prob and resid_mass are
                                 the fp64 evaluation's */

/* Inputs.  All pointers are DEVICE pointers owned by the caller, row-major,
 * read-only for the library, and must stay valid until the stream reaches the
 * end of the call.  Logit tensors need 4-byte alignment; the fast path needs
 * 16-byte alignment of both base pointers and V * sizeof(element) divisible by 16. */
typedef struct sv_inputs {
    int32_t B;                    /* requests, >= 0 (B = 0 is a no-op) */
    int32_t K;                    /* drafts per request, 1..SV_MAX_K */
    int32_t L;                    /* draft length, 1..SV_MAX_L */
    int32_t V;                    /* vocabulary size, 1..SV_MAX_V */
    int32_t dtype;                /* sv_dtype of both logit tensors */
    const void *target_logits;    /* [B][K][L+1][V] */
    const void *draft_logits;     /* [B][K][L][V] */
    const int32_t *draft_tokens;  /* [B][K][L], X[b][k][j] drawn from draft row j */
    const float *temperature;     /* [B], T_b > 0 */
    const float *u_accept;        /* [B][K][L], uniforms in [0, 1) */
    const float *u_correct;       /* [B], uniforms in [0, 1) */
    const void *row_stats;        /* optional [B][K][2L+1] node-row statistics (sv_row_stat,
                                     rows as in sv_outputs.row_lse), e.g. from spec_lm_head;
                                     when set the library streams no rows for statistics
                                     and runs one walk (no second round); NULL: computed */
} sv_inputs;

/* Statistics of one logit row l at its request's temperature T: shift M and
 * sum S = sum_v 2^((l_v - M) log2(e) / T), so that the temperature softmax is
 * pi(v) = 2^((l_v - M) log2(e) / T) / S. */
typedef struct sv_row_stat {
    float shift;
    float pad;
    double sum;
} sv_row_stat;

/* Outputs.  DEVICE pointers owned by the caller; every element of every
 * non-null output is overwritten.  The three integer outputs are required. */
typedef struct sv_outputs {
    int32_t *accept_len;   /* [B] tau in [0, L]; -1 for an invalid request */
    int32_t *draft_index;  /* [B] the draft whose prefix was accepted, -1 iff tau <= 0 */
    int32_t *correction;   /* [B] token id in [0, V); -1 for an invalid request */
    int32_t *flags;        /* optional [B]: SV_FLAG_* bits */
    float *row_lse;        /* optional [B][K][2L+1]: ln sum_v exp(l_v / T_b) of the node
                              row of (k, row); rows 0..L are target rows, L+1..2L
                              draft rows 0..L-1.  Requesting it makes the
                              statistics kernel stream every node row (one round,
                              target rows at position L included). */
    float *accept_prob;    /* optional [B][K][L]: h of each test evaluated exactly,
                              NaN where no test was made or where the test was
                              settled by the bound h <= w without computing h */
    float *resid_mass;     /* optional [B]: mass Z (in probability units) of the
                              distribution the correction was drawn from */
    int32_t *rows_streamed;/* optional [B]: logit rows whose softmax statistics the
                              row-statistics kernel computed for the request (its
                              algorithmic bytes are rows_streamed * V * sizeof(elem)) */
} sv_outputs;

/* Launch resources. */
typedef struct sv_launch {
    void *stream;          /* hipStream_t to launch on; NULL = the null stream */
    void *workspace;       /* device scratch, 256-byte aligned, contents need not
                              be initialised, >= sv_workspace_size(...) bytes */
    size_t workspace_bytes;
    void *phase_events[5]; /* optional hipEvent_t, recorded on `stream` when non-null:
                              [0] before the first row-statistics launch, [1] before the
                              first walk launch, [2] after it, [3] after the second
                              row-statistics launch, [4] after the second walk launch
                              (the second round runs only for K > 1 without
                              diagnostics; otherwise [2], [3], [4] coincide) */
} sv_launch;

/* Workspace bytes a call with these sizes needs (0 on invalid sizes): row
 * statistics (16 bytes per node row, reused after the walk for the fp64
 * statistics of the requests taken again), one saved walk state per request,
 * the rows listed for the second round, the list of requests taken again in
 * fp64 (4 bytes per request) and, for K >= 3, one node list per request
 * (196 608 bytes: the tokens a node's repeated residual-mass sweeps still need,
 * so those sweeps read a few thousand entries instead of two rows of V).  With
 * K = 1 the single-draft path's slice statistics, residual slice sums and
 * per-request chains when they are larger. */
size_t sv_workspace_size(int32_t B, int32_t K, int32_t L, int32_t V, int32_t dtype);

/* Token-level speculative sampling (K must be 1). */
int spec_verify_token(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln);

/* Greedy block verification of one draft (K must be 1). */
int spec_verify_block(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln);

/* Block verification over K i.i.d. drafts (K >= 1; K = 1 equals spec_verify_block). */
int spec_verify_multidraft(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln);

/* SpecTr over K i.i.d. drafts (K >= 1; K = 1 equals spec_verify_token).  Same
 * inputs, outputs, workspace and events as spec_verify_multidraft; accept_prob
 * holds h of every test made (NaN for drafts not tested). */
int spec_verify_spectr(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln);

/* SpecTr with rho* found by plain bisection of [1, n] (one sweep per halving,
 * to 1e-7 relative), the O(V log K) selection step the SpecTr-GBV page puts on
 * SpecTr (section 3) and measures its method against (section 4, time
 * efficiency).  Same rule, arguments and results as spec_verify_spectr, whose
 * search (a histogram sweep, then a few Newton sweeps) reaches the same rho* in
 * fewer sweeps. */
int spec_verify_spectr_bisect(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): spec_verify_multidraft
 * with the workspace taken from scratch memory the library holds itself, a
 * static device array of SV_NOALLOC_SCRATCH_BYTES on each device it is used on
 * (held until the process ends).  The call allocates nothing.  The caller still
 * passes inputs and outputs (device memory, as for spec_verify_multidraft);
 * `stream` is the hipStream_t to launch on (NULL = the null stream of the
 * current device), and the scratch of that stream's device is used.  Results
 * equal spec_verify_multidraft's.  Sizes whose workspace
 * (sv_workspace_size) exceeds SV_NOALLOC_SCRATCH_BYTES return SV_EUNSUPPORTED
 * before any launch; B = 512, K = L = 8 still fits, B = 1024, K = 4, L = 8 does
 * not.  Every call on one device shares that device's scratch: calls that can
 * overlap on one device (different streams, or different threads without
 * ordering) race and must not be issued; calls ordered on one stream are safe.
 * Phase events are not recorded. */
#define SV_NOALLOC_SCRATCH_BYTES (128u << 20)
int spec_verify_multidraft_noalloc(const sv_inputs *in, const sv_outputs *out, void *stream);

/* ------------------------------------------------------------- drafting */

/* Drafting: the other half of the draft-then-verify loop (MineDraft page,
 * section 1; SpecTr-GBV page, section 2, step 1: K i.i.d. draft blocks of
 * length L).  Given the draft model's logits, draw the blocks position by
 * position: draft k draws X[b][k][j] from the temperature softmax of the node
 * row of its prefix X[b][k][0..j-1] -- the row of the lowest-index draft with
 * that prefix, the node rule the verifier uses, so drafts that meet at a node
 * draw from one distribution and a caller may leave the other rows unwritten --
 * by the inverse CDF of u_draft[b][k][j]: y = min{v : C_v > u Z} in token-id
 * order (the last token of positive weight if rounding leaves none).  Each
 * draft's block is then an independent draw.  Tokens match the CPU oracle
 * except where u Z lies within ~1e-6 Z of a CDF boundary. */
typedef struct sv_draft_inputs {
    int32_t B, K, L, V;           /* as in sv_inputs */
    int32_t dtype;                /* sv_dtype of the logits */
    const void *draft_logits;     /* [B][K][L][V], device memory */
    const float *temperature;     /* [B], T_b > 0 */
    const float *u_draft;         /* [B][K][L], uniforms in [0, 1) */
} sv_draft_inputs;

typedef struct sv_draft_outputs {
    int32_t *draft_tokens;        /* [B][K][L], required; all -1 for an invalid request
                                     (T not positive finite, a uniform outside [0, 1),
                                     or a node row read that is not a distribution) */
    int32_t *flags;               /* optional [B]: SV_FLAG_INVALID or 0 */
    int32_t *rows_streamed;       /* optional [B]: node rows read */
} sv_draft_outputs;

/* Workspace bytes spec_draft_sample needs (0 on invalid sizes). */
size_t sv_draft_workspace_size(int32_t B, int32_t K, int32_t L, int32_t V, int32_t dtype);

/* Draw the K draft blocks of every request.  Asynchronous on ln->stream:
 * per position, list the node rows, stream them into tile sums and draw (with
 * K <= 16 the draw of position j also lists the node rows of position j + 1:
 * 2L + 3 launches in all, else 3L + 2), plus a clear and a final pass that
 * marks invalid requests.  ln->phase_events[0] and [1], when non-null, are
 * recorded before and after them; [2..4] are not used.  The tokens of position j are written by
 * the launch for j and read back by the later ones, so draft_tokens must not
 * alias the other arguments. */
int spec_draft_sample(const sv_draft_inputs *in, const sv_draft_outputs *out,
                      const sv_launch *ln);

/* ------------------------------------------------------- fused LM head */

/* The step that produces the verifier's inputs: logits = h W^T for bf16 hidden
 * states h [R][d] and a bf16 vocabulary projection W [V][d] (row-major, so both
 * operands are contiguous along d), fp32 accumulation on the matrix cores, fp32
 * or bf16 logits out.  The temperature-softmax statistics of every row (the verifier's
 * first step) are computed in the same kernel while the row is in registers,
 * so passing them to a verification call (sv_inputs.row_stats) removes the
 * statistics pass over the logits.  Verification is a large share of a
 * speculative-decoding step (the performance study's page, section 1). */
typedef struct sv_lm_inputs {
    int32_t R;                    /* rows, >= 0 */
    int32_t d;                    /* hidden size, a multiple of 64, 128 <= d <= 65536 */
    int32_t V;                    /* vocabulary size, 1..SV_MAX_V */
    const void *hidden;           /* [R][d] bf16, 16-byte aligned, device memory */
    const void *weight;           /* [V][d] bf16, 16-byte aligned, device memory */
    const float *temperature;     /* [R]: the temperature of each row's request */
} sv_lm_inputs;

typedef struct sv_lm_outputs {
    void *logits;                 /* [R][V], required: fp32, or bf16 when logits_dtype is
                                     SV_BF16 (rounded to nearest even; the statistics are
                                     then those of the rounded values, as the verifier
                                     reads them) */
    void *row_stats;              /* optional sv_row_stat array: row r is written to slot
                                     (r / stats_group) * stats_stride + stats_offset
                                     + r % stats_group.  Target rows [B][K][L+1] go to
                                     group L+1, stride 2L+1, offset 0; draft rows
                                     [B][K][L] to group L, stride 2L+1, offset L+1. */
    int32_t stats_group, stats_stride, stats_offset;
    int32_t logits_dtype;         /* SV_F32 or SV_BF16 */
} sv_lm_outputs;

/* Workspace bytes spec_lm_head needs (0 on invalid sizes). */
size_t sv_lm_workspace_size(int32_t R, int32_t d, int32_t V);

/* Compute the logits (and statistics) asynchronously on ln->stream; events [0]
 * and [1], when non-null, are recorded before and after. */
int spec_lm_head(const sv_lm_inputs *in, const sv_lm_outputs *out, const sv_launch *ln);

/* Static description of a status code. */
const char *sv_status_string(int status);

/* Library version, e.g. "0.2.0". */
const char *sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
