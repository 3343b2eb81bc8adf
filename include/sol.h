/*
 * sol.h -- C ABI of the Sol-Attn library for MI355X (gfx950), libsol.so.
 *
 * Sol-Attn ("Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
 * Attention Sparsification"; abstract and the "Sol-Attn" visual paper
 * explainer) computes block-sparse attention in one online-softmax sweep:
 * pool Q, K and V into blocks; compare each pooled-key proxy score with a
 * per-query-block threshold tau = mu + beta*sigma; compute selected key
 * blocks exactly and fold every unselected block in as one pooled key that
 * stands for its tokens, with their summed values.
 *
 * Conventions shared by every entry point:
 *  - Token tensors q, k, v, out are DEVICE pointers to [H][L][d] row-major,
 *    contiguous arrays of `dt` elements (bf16 or fp32), 16-byte aligned.
 *    The caller owns all memory; the library allocates nothing (apart from
 *    the static scratch of sol_attn_fwd_noalloc, see there).
 *  - Blocks are B consecutive tokens; N = ceil(L / B); the last block holds
 *    n_last = L - (N-1)*B valid tokens and is masked, never padded.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on that stream: it validates its arguments on the host,
 *    enqueues kernels and returns.  Device-side faults surface at the
 *    caller's next synchronisation of the stream.
 *  - Return value: SOL_OK, or a negative sol_status_t.  Argument errors are
 *    detected before anything is enqueued, and nothing is written then.
 *  - Supported shapes: d in {64, 128}, B in {32, 64, 128}, H >= 1, 1 <= L and
 *    N <= 8192; anything else returns SOL_EUNSUPPORTED.
 *  - Calls that share a workspace must be ordered on one stream; concurrent
 *    calls need distinct workspaces.
 */
#ifndef SOL_H
#define SOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SOL_BF16 = 0, SOL_F32 = 1 } sol_dtype_t;

typedef enum {
    SOL_OK = 0,
    SOL_EINVAL = -1,        /* null pointer, non-positive size, NaN beta, bad dtype */
    SOL_EUNSUPPORTED = -2,  /* d, B or N outside the supported set */
    SOL_EWORKSPACE = -3,    /* workspace missing or smaller than sol_workspace_bytes */
    SOL_EHIP = -4,          /* a HIP launch or query failed */
    SOL_ESCRATCH = -5       /* sol_attn_fwd_noalloc: the shape needs more than its static scratch */
} sol_status_t;

/*
 * Bytes of device workspace sol_attn_fwd / sol_attn_fwd_dbg (and sol_route,
 * sol_sweep) need for this shape: the pooled tensors (3 x H*N*d fp32), the
 * per-query-block thresholds (H*N fp32), the scheduler's queue counters, bf16
 * copies of the pooled keys and summed values (2 x H*N*d bf16), the
 * selection bits (H*N*ceil(N/32) uint32) and the key moments
 * (H*(d + d*d) fp32).  0 for invalid shapes.
 */
size_t sol_workspace_bytes(int H, int L, int d, int B);

/*
 * Block pooling ("Sol-Attn" visual explainer, "Pool Q, K and V into blocks";
 * Eq. (5) legend: the mean query and key vector of a block; Eq. (10) legend:
 * the summed values).  For each head h and block j, over its n_j valid
 * tokens:
 *     qbar[h][j] = mean of q,  kbar[h][j] = mean of k,  vsum[h][j] = sum of v.
 * qbar, kbar, vsum: DEVICE fp32 [H][N][d], written entirely.
 */
int sol_pool(const void* q, const void* k, const void* v,
             int H, int L, int d, int B, sol_dtype_t dt,
             float* qbar, float* kbar, float* vsum, void* stream);

/*
 * Routing statistics ("Sol-Attn" visual explainer, Eq. (4) and Eq. (5);
 * Eq. (11) right-hand side for the proxy score).  For every (h, i):
 *     s_ij  = qbar_i . kbar_j / sqrt(d)  for j = 0..N-1 (kept on chip only)
 *     mu_i  = (1/N) sum_j s_ij,  sigma_i^2 = (1/N) sum_j (s_ij - mu_i)^2
 *     tau_i = mu_i + beta * sigma_i      (beta = -inf / +inf -> tau = -inf / +inf)
 *     kept_counts[h][i] = |{ j : s_ij > tau_i }|
 * qbar, kbar : DEVICE fp32 [H][N][d] (as written by sol_pool).
 * tau        : DEVICE fp32 [H][N], written.
 * kept_counts: DEVICE int32 [H][N], written.
 * sel_bits   : DEVICE uint32 [H][N][ceil(N/32)], written, or NULL: the
 *              decisions themselves, bit (j % 32) of word j / 32 of row (h, i)
 *              set iff s_ij > tau_i (the layout of sol_attn_fwd_dbg's
 *              sel_mask).  sol_sweep can take them instead of deriving them.
 * workspace  : DEVICE, at least sol_workspace_bytes(H, L, d, B) bytes,
 *              256-byte aligned (scratch; missing or small: SOL_EWORKSPACE).
 * For N <= 1280 each row s_i. is held on chip and mu_i, sigma_i are its
 * two-pass statistics.  For longer rows mu_i and sigma_i come from the key
 * moments of Eq. (5), taken about the mean pooled key (equal in exact
 * arithmetic): mu_i = c qbar_i . mbar and sigma_i^2 = c^2 qbar_i Cov qbar_i^T
 * with mbar = (1/N) sum_j kbar_j and Cov = (1/N) sum_j (kbar_j - mbar)
 * (kbar_j - mbar)^T (summed in fp64 into the workspace as fp32; no
 * subtraction of nearly equal terms when the keys share a large common
 * component; mu_i, sigma_i and tau_i in fp64, tau_i rounded to fp32).  A row whose
 * sigma_i is 0 (all its scores equal) keeps no block: none is strictly above
 * tau_i = mu_i.
 * The counts and bits are those the forward pass uses (the same kernels
 * form every s_ij: fp32 matrix instructions for N <= 1280, three-way bf16
 * splits of the fp32 vectors, at fp32 accuracy, for longer rows; both
 * sweeps take their decisions from these bits).
 */
int sol_route(const float* qbar, const float* kbar, int H, int L, int d, int B,
              float beta, float* tau, int32_t* kept_counts, uint32_t* sel_bits,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * The fused sweep alone: given the pooled tensors and thresholds, route each
 * key block of every (h, i) (s_ij > tau_i: exact; otherwise approximate) and
 * merge both paths into one online softmax ("Sol-Attn" visual explainer,
 * Eq. (9), Eq. (10), Eq. (11); abstract).  Output as sol_attn_fwd.
 * qbar, kbar, vsum : DEVICE fp32 [H][N][d] as written by sol_pool.
 * tau       : DEVICE fp32 [H][N] as written by sol_route.
 * workspace : DEVICE, at least sol_workspace_bytes(H, L, d, B) bytes,
 *             256-byte aligned (scratch: work counters, bf16 copies of the
 *             pooled keys and summed values, and the query-block grouping
 *             costs and strides; see sol_attn_fwd).
 * sel_bits  : DEVICE, the decisions sol_route wrote for these thresholds, or
 *             NULL.  When given, the sweep takes its decisions from them and
 *             launches no routing pass of its own; when NULL it first derives
 *             them from tau.
 * sel_mask  : as in sol_attn_fwd_dbg (the decisions taken), or NULL.
 */
int sol_sweep(const void* q, const void* k, const void* v,
              const float* qbar, const float* kbar, const float* vsum, const float* tau,
              int H, int L, int d, int B, sol_dtype_t dt, void* out,
              void* workspace, size_t ws_bytes, const uint32_t* sel_bits,
              uint32_t* sel_mask, void* stream);

/*
 * sol_sweep (bf16, with the caller's selection bits) for scheduling
 * measurements: the same kernel, recording for every group item when a
 * workgroup claimed it and when it finished, and optionally claiming items
 * in a caller-given order instead of from the per-XCD queues.  The abstract
 * notes that selection gives query blocks "dynamic but potentially
 * imbalanced budgets"; this measures what the claim order does about it.
 * A group item is one workgroup's 128 / B query blocks of one head: item
 * h * G + g for g < G = ceil(N / (128 / B)) (B = 64: pairs of query blocks;
 * which blocks form group g depends on the head's group stride, chosen from
 * the selection: see sol_attn_fwd).
 * order      : DEVICE int32 [H*G], a permutation of 0 .. H*G-1 (claimed in
 *              that order by one counter), or NULL for the per-XCD queues.
 *              An entry outside 0 .. H*G-1 ends the claiming workgroup.
 * item_clock : DEVICE uint64 [H*G][3], written: claim time, end time (the
 *              100 MHz constant clock of s_memrealtime) and workgroup index.
 * Other arguments as sol_sweep (sel_bits required).  Outputs are those of
 * sol_sweep for the same selection (bit for bit with order NULL).
 * Errors: as sol_sweep; fp32 inputs: SOL_EUNSUPPORTED.
 */
int sol_sweep_timed(const void* q, const void* k, const void* v,
                    const float* qbar, const float* kbar, const float* vsum, const float* tau,
                    int H, int L, int d, int B, sol_dtype_t dt, void* out,
                    void* workspace, size_t ws_bytes, const uint32_t* sel_bits,
                    const int32_t* order, uint64_t* item_clock, void* stream);

/*
 * Sol-Attn forward ("Sol-Attn" visual explainer: Eq. (4) selection rule,
 * Eq. (5) statistics over all N key blocks, Eq. (9) denominator, Eq. (10)
 * numerator, Eq. (11) token-to-pooled-block tile; abstract: one
 * online-softmax pass without materialising the proxy map).  For each head h
 * and query block i:
 *     s_ij  = qbar_i . kbar_j / sqrt(d)        for all key blocks j
 *     tau_i = mu_i + beta * sigma_i            (population mean / std of s_i.)
 *     S_i   = { j : s_ij > tau_i }             (strict; beta=-inf: all, +inf: none)
 * and for every query token r of block i, with a = q_r.k_t/sqrt(d) for keys
 * t of selected blocks and g_j = q_r.kbar_j/sqrt(d) for unselected blocks j:
 *     out_r = (sum_{j in U} e^{g_j} vsum_j + sum_{S} sum_t e^{a} v_t)
 *           / (sum_{j in U} n_j e^{g_j}   + sum_{S} sum_t e^{a})
 * Proxy scores exist only on chip; they are never written to memory.
 * Equivalent to sol_pool, then sol_route, then sol_sweep on one stream.
 * Work layout (bf16 sweep): query blocks go in groups of 128 / B that share
 * one list of key tiles, the union of their selections.  Per head a group
 * holds consecutive blocks, or blocks spaced by a group stride s in 2..8
 * (runs of (128 / B) s blocks, group r of a run holding blocks r, r + s, ...;
 * consecutive groups after the last whole run) when that stride gives the
 * smallest summed union size (ties: the smaller stride).  The grouping
 * changes only the order in which a row's terms are accumulated.
 *
 * beta        : any float except NaN (+-INFINITY allowed).
 * out         : DEVICE [H][L][d], dtype dt.
 * kept_counts : DEVICE int32 [H][N], |S_i| for every (h, i).
 * workspace   : DEVICE, at least sol_workspace_bytes(H, L, d, B) bytes,
 *               256-byte aligned; contents are scratch (no state is kept
 *               between calls).
 */
int sol_attn_fwd(const void* q, const void* k, const void* v,
                 int H, int L, int d, int B, float beta, sol_dtype_t dt,
                 void* out, int32_t* kept_counts,
                 void* workspace, size_t ws_bytes, void* stream);

/*
 * sol_attn_fwd plus diagnostics, for parity checks (never in timed runs):
 * sel_mask : DEVICE uint32 [H][N][ceil(N/32)] or NULL; bit (j % 32) of word
 *            j / 32 of row (h, i) is 1 iff key block j was computed exactly.
 *            These are the decisions the attention kernel itself took.
 * tau      : DEVICE fp32 [H][N] or NULL; the thresholds tau_i used.
 */
int sol_attn_fwd_dbg(const void* q, const void* k, const void* v,
                     int H, int L, int d, int B, float beta, sol_dtype_t dt,
                     void* out, int32_t* kept_counts,
                     void* workspace, size_t ws_bytes, void* stream,
                     uint32_t* sel_mask, float* tau);

/*
 * The forward pass with the comparators the pages contrast Sol-Attn with,
 * for accuracy studies (abstract: routing that gives every query block the
 * same share of top-scoring key blocks, and keep-or-drop sparsification that
 * discards what is not selected; visual explainer, "Place it among nearby
 * methods": ordinary block sparse attention lets every unselected block
 * contribute zero).  flags is a bitwise OR of:
 *   SOL_DROP_APPROX  unselected blocks contribute nothing (no Eq. (9) /
 *                    Eq. (10) approximate terms); a row whose selection is
 *                    empty is written as zeros.
 *   SOL_TOPK         every query block selects the k = round(keep_frac * N)
 *                    blocks (halves up, within [0, N]) with the largest proxy
 *                    scores, ties to the lower block index, instead of
 *                    s_ij > tau_i; beta is ignored, tau receives the k-th
 *                    largest score (+inf for k = 0) and kept_counts = k.
 *   SOL_FUSED_ROUTE  the routing as the pages' fused kernel does it ("Sol-Attn"
 *                    visual explainer, "How the fused kernel executes it",
 *                    Eq. (11); Eq. (5)): the thresholds come first, from the
 *                    Eq. (5) key moments (mean pooled key and covariance about
 *                    it, fp64) for every N, and no decision is computed or
 *                    stored before the sweep; each workgroup forms its query
 *                    blocks' proxy scores qbar_i . kbar_j / sqrt(d) in fp32, 32
 *                    key blocks at a time, compares them with tau_i, builds its
 *                    tile list from those decisions and writes its kept
 *                    counts.  No decision map exists in device memory unless
 *                    sel_mask asks for it.  Decisions agree with the default
 *                    route except within fp32 rounding of tau_i; query blocks
 *                    are grouped consecutively.  Not with SOL_TOPK.
 * flags = 0 is sol_attn_fwd_dbg.  Other arguments as sol_attn_fwd_dbg.
 * Errors: unknown flag bits, SOL_TOPK with SOL_FUSED_ROUTE, or SOL_TOPK with
 * keep_frac outside [0, 1] or NaN: SOL_EINVAL; nonzero flags with SOL_F32:
 * SOL_EUNSUPPORTED.
 */
#define SOL_DROP_APPROX 1u
#define SOL_TOPK 2u
#define SOL_FUSED_ROUTE 4u
int sol_attn_fwd_variant(const void* q, const void* k, const void* v,
                         int H, int L, int d, int B, float beta, float keep_frac,
                         unsigned flags, sol_dtype_t dt, void* out, int32_t* kept_counts,
                         void* workspace, size_t ws_bytes, void* stream,
                         uint32_t* sel_mask, float* tau);

/*
 * Dense softmax attention softmax(Q K^T / sqrt(d)) V (the pages' speedup
 * baseline, "Sol-Attn" visual explainer, "What the paper measured": dense
 * attention wall time over the method's), on the same tile machinery with
 * every key block computed exactly.  out: DEVICE [H][L][d], dtype dt.
 * Needs no workspace.  d in {64, 128}.
 */
int sol_attn_dense(const void* q, const void* k, const void* v,
                   int H, int L, int d, sol_dtype_t dt, void* out, void* stream);

/*
 * sol_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: its workspace is
 * a static device array of SOL_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on, from its first use there until the process ends.
 * Results are those of sol_attn_fwd (the same kernels).
 *
 * Arguments as sol_attn_fwd; the kernels run on `stream`, whose device's
 * copy of the scratch they use (the current device for the NULL stream).
 * Errors: as sol_attn_fwd; SOL_ESCRATCH when the shape needs more scratch
 * than SOL_NOALLOC_SCRATCH_BYTES, checked on the host before anything is
 * enqueued.  The scratch holds, each region rounded up to 256 bytes: the
 * pooled values (bf16 inputs: two fp32 and two bf16 copies of H*N*d values;
 * fp32 inputs: three fp32 and two bf16), the thresholds (H*N fp32), the
 * selection bits (H*N*ceil(N/32) uint32) and the key moments
 * (H*(d + d*d) fp32).  The Wan-2.1-shaped layer (40 heads, 75,600 tokens,
 * d = 128, B = 64, bf16) needs 82.5 MB of the 96 MiB.
 * Calls on one GPU share its scratch: calls that may overlap in time on one
 * GPU (on different streams, or from different threads) race and give
 * undefined results; order them on one stream or use sol_attn_fwd with
 * distinct workspaces.
 */
#define SOL_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int sol_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                         int H, int L, int d, int B, float beta, sol_dtype_t dt,
                         void* out, int32_t* kept_counts, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* sol_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SOL_H */
