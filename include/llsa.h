/*
 * llsa.h -- C ABI of the MI355X (gfx950) Log-linear Sparse Attention hot path.
 *
 * Source of the method: the pith.science review page of arXiv 2512.16615, "Trainable Log-linear
 * Sparse Attention for Efficient Diffusion Transformers" (cited below as "LLSA review").  The
 * problem is stated there as sparse attention on Q, K, V with a block size B, a Top-K parameter K,
 * L pooled levels and L_e enrichment levels (parameter ledger; Figure 1 caption).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are device pointers into caller-owned memory.  Raw tensors Q, K, V, O, dO, dQ, dK, dV are
 * [batch][heads][n][d], contiguous, d fastest, stored as fp32 or bf16 (llsa_problem.dtype).
 * The pooled pyramid is fp32 [batch*heads][R][d] with R = sum_{l=1..L} n_l and n_l = n / B^l; level l
 * starts at row sum_{l'<l} n_l'.  Selection indices are int32 [batch*heads][R][K] (same row order), each row
 * ascending.
 * Pooled K and V in the attention calls (an amendment of the five-call contract, which passes the fp32
 * pyramids): llsa_attn_fwd and llsa_attn_bwd read the pooled K and V pyramids in the raw dtype -- the fp32
 * pyramids themselves for fp32 problems; for bf16 problems their bf16 copies (same layout, rounded to nearest
 * even), which llsa_build_pyramid writes beside the fp32 pyramids (pk_bf16, pv_bf16).  The bf16 products round
 * pooled tokens to bf16 anyway, so the copies change no result; reading fp32 rows instead doubles the bytes
 * of every enrichment gather, measured on MI355X as one more 32-entry stage per fine block: +48 us per step at
 * n = 65536, 16 heads, K = 8, L = 3 (0.873 -> 0.921 ms: forward +20 us, dQ +32 us) and +0.10 ms at n = 262144,
 * 8 heads, K = 16 (2.76 -> 2.86 ms), with identical outputs.
 * Index inputs: every idx passed to a call must be a selection as llsa_select writes it -- values of level l in
 * [0, n_l), rows ascending, each unit's picks children of its parent's picks.  The attention calls gather rows
 * at those indices without checking them: any other idx is undefined behaviour (an out-of-range value reads
 * outside the tensors).  The transposes skip negative and clamp too-large values, so they never write outside
 * their arrays, but their result for such an idx is unspecified.  The CSC of level l (l = 1..T, T = max(1, L_e)) is col_ptr (n_l + 1 entries,
 * relative to the level) and perm (n_l * K entries, each a CSR position p = u*K + k, ascending within
 * a column); levels are concatenated per batch*head in level order.
 *
 * Ownership: the caller allocates and owns every buffer, including workspaces; the library allocates
 * nothing on these paths, keeps no pointer after returning and holds no state beyond a cached
 * per-device property query (and, only while llsa_timing_enable is on, its timing events).  Calls are
 * re-entrant.
 * Asynchrony: each call validates on the host, then enqueues kernels on `stream` (a hipStream_t;
 * NULL means the default stream) and returns without synchronising.  Outputs are complete when the
 * stream reaches that point; they are overwritten, never accumulated.
 * Errors: each call returns LLSA_OK (0) or a negative LLSA_ERR_* code; on a validation error nothing
 * is launched.  No exception crosses the ABI.  Non-finite inputs give unspecified outputs.
 * Pointers must be 16-byte aligned (LLSA_ERR_ALIGN).
 * GPU limits of this version: d = 64, B = 16, 1 <= K <= n_L, K <= 32, n_L <= 512, K*L_e <= 128,
 * K*(L_e-1) <= 32 for the backward, batch*heads*n*d < 2^31.
 */
#ifndef LLSA_H
#define LLSA_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLSA_F32 = 0, LLSA_BF16 = 1 } llsa_dtype;

enum {
  LLSA_OK = 0,
  LLSA_ERR_NULL = -1,        /* a required pointer is NULL                                        */
  LLSA_ERR_SHAPE = -2,       /* n mod B^L != 0, L or K or L_e out of range, bad batch/heads/n     */
  LLSA_ERR_UNSUPPORTED = -3, /* valid for the method but outside this GPU version (d, B, sizes)   */
  LLSA_ERR_DTYPE = -4,       /* unknown dtype, or a dtype an entry point does not implement      */
  LLSA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                                  */
  LLSA_ERR_WORKSPACE = -6,   /* workspace pointer NULL or ws_bytes smaller than required          */
  LLSA_ERR_LAUNCH = -7,      /* a kernel launch failed (hipGetLastError)                           */
  LLSA_ERR_PARAM = -8,       /* scale not finite                                                   */
  LLSA_ERR_DEVICE = -9,      /* current device is not gfx950                                       */
  LLSA_ERR_SCRATCH = -10     /* the problem needs more than the static scratch of a no-alloc call   */
};

/* Problem description; every entry point takes the same struct. */
typedef struct {
  int32_t batch, heads, n, d; /* raw tensors [batch][heads][n][d]                                  */
  int32_t block;              /* B: pooling factor and attention block size                          */
  int32_t topk;               /* K: blocks kept per query unit at every level                        */
  int32_t levels;             /* L; 0 selects floor(log_B n - 1) [LLSA review, parameter ledger]     */
  int32_t enrich_levels;      /* L_e in [0, L]; -1 selects L [LLSA review, parameter ledger]         */
  int32_t dtype;              /* llsa_dtype of the raw tensors                                        */
  float scale;                /* softmax scale sigma; 0 selects 1/sqrt(d)                             */
  int32_t grid_w;             /* scheduling hint: tokens per row when each slice is a row-major 2-D    */
                              /* token grid (n = rows * grid_w), else 0; used when grid_w is a multiple */
                              /* of 4B that divides n, ignored otherwise; negative: LLSA_ERR_SHAPE.     */
                              /* With it, the bf16 forward pairs each fine block with the one a grid    */
                              /* row below (their selections overlap) where it pairs neighbours         */
                              /* without, and the dK/dV work list takes key-block groups of four        */
                              /* consecutive grid rows together (they share query blocks).  The         */
                              /* selection never depends on it, and neither does the backward given the */
                              /* same forward outputs; the bf16 forward's O and LSE differ only by the   */
                              /* order of its floating-point sums (within the bf16 tolerance).          */
} llsa_problem;

/* Operation ids for llsa_workspace_bytes. */
enum {
  LLSA_OP_INDEX_TRANSPOSE = 1,
  LLSA_OP_ATTN_BWD = 2,
  LLSA_OP_ATTN_FWD_COMPLEMENT = 3,
  LLSA_OP_ATTN_BWD_COMPLEMENT = 4
};

/*
 * llsa_build_pyramid -- hierarchical compression [LLSA review, "Core claim"; "What carries the
 * argument"]: X^(l)[j] = mean of B consecutive tokens of X^(l-1), l = 1..L, X^(0) = X, for X in
 * {Q, K, V}.  Accumulation and storage in fp32.
 *   q, k, v   in : raw tensors (dtype).
 *   pq, pk, pv out: fp32 pyramids [batch*heads][R][d].
 *   pk_bf16, pv_bf16 out (bf16 problems; ignored and may be NULL for fp32): the pooled K and V pyramids
 *             rounded to bf16 (round to nearest even), bf16 [batch*heads][R][d] -- the pyramid operands of
 *             llsa_attn_fwd / llsa_attn_bwd, whose bf16 products round pooled tokens to bf16.  These two
 *             parameters extend the five-call contract (see "Pooled K and V in the attention calls" above).
 */
int llsa_build_pyramid(const llsa_problem* prob, const void* q, const void* k, const void* v, float* pq,
                       float* pk, float* pv, void* pk_bf16, void* pv_bf16, hipStream_t stream);

/*
 * llsa_select -- hierarchical Top-K [LLSA review, "Core claim"; "What carries the argument";
 * referee major comment 1 on Algorithm 1]: every level-L unit scores all n_L pooled key blocks with
 * the dot product of pooled query and pooled key and keeps the best K; at l = L-1..1 unit u scores
 * only the B children of each block its parent u/B kept and keeps the best K.  Ties go to the lower
 * block index.  Scores are computed in fp32.
 *   pq, pk in : fp32 pyramids from llsa_build_pyramid.
 *   idx    out: int32 [batch*heads][R][K], each row ascending.
 */
int llsa_select(const llsa_problem* prob, const float* pq, const float* pk, int32_t* idx, hipStream_t stream);

/*
 * llsa_select_exhaustive -- single-level exhaustive Top-K, the quadratic baseline the hierarchy replaces
 * [LLSA review, Figure 1 caption (general Top-K) and referee major comment 2 (routing recall of the
 * hierarchical selection)]: every level-1 unit scores all n_1 level-1 pooled key blocks (unscaled pooled
 * query . pooled key, fp32) and keeps the best K, ties to the lower block index, each row ascending.  Not part
 * of the hot path; used to measure how many of the exhaustive picks the hierarchy finds.
 *   pq, pk in : fp32 pyramids from llsa_build_pyramid (only level 1 is read).
 *   idx1   out: int32 [batch*heads][n_1][K].
 * Limits as llsa_select, except that n_1 is not limited by n_L <= 512.
 */
int llsa_select_exhaustive(const llsa_problem* prob, const float* pq, const float* pk, int32_t* idx1, hipStream_t stream);

/*
 * llsa_reorder -- 2-D-local index reordering of the token rows [LLSA review, domain-assumption ledger: after
 * index reordering spatially adjacent pixels are adjacent in the sequence (paper Sec. 5.1, ablation Table 5d);
 * Figure 2 caption].  The page does not give the order; this one takes recursive 4 x 4 tiles, so that every
 * level-l unit (16^l consecutive tokens) is a 4^l x 4^l pixel patch for l <= L: pixel (y, x) of the row-major
 * grid goes to (row-major index of its 4^L x 4^L top tile) * 16^L + sum_{k<L} (4 digit_k(y) + digit_k(x)) 16^k,
 * digit_k the k-th base-4 digit of the coordinate inside the top tile.  Applied before the path to Q, K, V
 * (and dO), and with to_local = 0 after it to O (and dQ, dK, dV).
 *   grid_h, grid_w: the pixel grid, grid_h * grid_w = n, both divisible by 4^L (LLSA_ERR_SHAPE otherwise).
 *   to_local: non-zero: row-major -> local order; zero: local -> row-major.
 *   x in, y out: raw tensors [batch][heads][n][d] (dtype), distinct buffers (LLSA_ERR_PARAM if x == y).
 */
int llsa_reorder(const llsa_problem* prob, int32_t grid_h, int32_t grid_w, int32_t to_local, const void* x, void* y,
                 hipStream_t stream);

/*
 * llsa_attn_fwd -- sparse block attention with hierarchical KV enrichment [LLSA review, "Core
 * claim"; "What carries the argument"; abstract]: raw query t in fine block i = t/B attends the B
 * raw tokens of every level-1 block in idx row i (logit sigma*q.k) and, for l = 1..L_e, the level-l
 * pooled tokens kept by its level-l ancestor unit i/B^(l-1) (logit sigma*q.k + l*ln B, i.e. weight
 * B^l).  Only the sparse indices are read; no dense mask exists.
 *   q, k, v in : raw tensors (dtype).  idx in: from llsa_select (any other idx: undefined behaviour).
 *   pk, pv  in : pooled K and V pyramids in the raw dtype (fp32: pk, pv of llsa_build_pyramid; bf16: its
 *                pk_bf16, pv_bf16 -- the amendment described above).
 *   o   out: [batch][heads][n][d] (dtype).
 *   lse out: fp32 [batch*heads][n], natural-log log-sum-exp of each query's logits (for backward).
 * bf16 runs the products on bf16 MFMA with fp32 accumulation (pooled K/V in bf16, probabilities rounded
 * to bf16 for the PV product); fp32 computes in fp32.
 */
int llsa_attn_fwd(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* pk,
                  const void* pv, const int32_t* idx, void* o, float* lse, hipStream_t stream);

/*
 * llsa_attn_fwd_complement -- the forward under the complement-partition reading of the enrichment, the
 * alternative the pages leave open [LLSA review, "Core claim" (enrichment appends coarse tokens, weight
 * B^l) and "What carries the argument" (O(K log N) tokens per query)]: raw query t in fine block i attends
 * the B raw tokens of every level-1 block in idx row i and, for l = 1..L_e, the level-l pooled tokens of the
 * blocks its level-l ancestor unit i/B^(l-1) scored but did not keep -- the B children of each block kept by
 * the unit's parent, or every block at the coarsest level -- with logit sigma*q.k + l*ln B.  With L_e = L
 * every raw key enters exactly once, as itself or through its finest scored-and-unkept ancestor.
 *   q, k, v, pk, pv, idx, o, lse: as llsa_attn_fwd (bf16 only: LLSA_ERR_DTYPE for fp32).
 *   idx must come from llsa_select (a hierarchical selection).
 *   ws scratch of llsa_workspace_bytes(prob, LLSA_OP_ATTN_FWD_COMPLEMENT) bytes (caller-owned): the
 *      complement lists, int32.
 * Limit: at most 576 entries per fine block, sum_{l<L} (B-1) K + (n_L - K) over l <= L_e
 * (LLSA_ERR_UNSUPPORTED otherwise); N = 262144, K = 16, L = 3 has 528.
 */
int llsa_attn_fwd_complement(const llsa_problem* prob, const void* q, const void* k, const void* v,
                             const void* pk, const void* pv, const int32_t* idx, void* o, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * llsa_attn_bwd_complement -- the backward of llsa_attn_fwd_complement [LLSA review, "If this is right" (the
 * backward uses only the sparse indices) and "Core claim" (pooled tokens, weight B^l)]: dQ, dK, dV through the
 * same entry sets; a level-l pooled token's gradient reaches each of the B^l raw tokens it averages with factor
 * B^-l.  Every gradient element is summed in a fixed order (bitwise reproducible).
 *   q, k, v, o, lse, dout, pk, pv, idx, dq, dk, dv: as llsa_attn_bwd (bf16 only), with o and lse from
 *      llsa_attn_fwd_complement; idx from llsa_select.
 *   ws scratch of llsa_workspace_bytes(prob, LLSA_OP_ATTN_BWD_COMPLEMENT) bytes (caller-owned): the complement
 *      lists, the CSC of levels 1..min(L_e + 1, L) (built here), Delta, per-level pooled gradients and their
 *      partial sums (fp32, 512 bytes per candidate per 256 queries).
 * Limit: as llsa_attn_fwd_complement (LLSA_ERR_UNSUPPORTED).
 */
int llsa_attn_bwd_complement(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* pk, const void* pv,
                             const int32_t* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * llsa_index_transpose -- CSR -> CSC of the selection of levels 1..T, T = max(1, L_e) [LLSA review,
 * "What carries the argument": a CSR-to-CSC scan gives each key block its query blocks without a
 * dense N x N mask].  Column j of level l lists the CSR positions p = u*K + k with idx = j, ascending.
 *   idx     in : from llsa_select (other values: skipped below 0, clamped above n_l - 1, result unspecified).
 *   col_ptr out: int32 [batch*heads][llsa_colptr_len].
 *   perm    out: int32 [batch*heads][llsa_perm_len].
 *   ws      scratch of llsa_workspace_bytes(prob, LLSA_OP_INDEX_TRANSPOSE) bytes (caller-owned).
 */
int llsa_index_transpose(const llsa_problem* prob, const int32_t* idx, int32_t* col_ptr, int32_t* perm,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llsa_index_transpose_noalloc -- for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): llsa_index_transpose with the same inputs, outputs and
 * result, its workspace taken from a library-owned static device array of LLSA_NOALLOC_SCRATCH_BYTES bytes
 * instead of a caller buffer.  Allocates nothing (no hipMalloc, hipFree or allocating library call); the
 * array's device address is looked up once per device, on the first call with that device current.
 *   idx, col_ptr, perm: as llsa_index_transpose.
 * Errors: as llsa_index_transpose, plus LLSA_ERR_SCRATCH (nothing launched) when
 * llsa_workspace_bytes(prob, LLSA_OP_INDEX_TRANSPOSE) exceeds LLSA_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. batch*heads =
 * 16 at n = 65536, K = 8 needs 2.5 MB; batch*heads = 8 at n = 262144, K = 16 needs 9.5 MB).
 * Every call on one GPU uses that GPU's single array, which keeps the last call's contents (the kernels clear
 * what must start at zero themselves): calls that overlap in time on one GPU -- on different streams, or from
 * different host threads -- race and give undefined results.  Serialise them (one stream, or events).
 */
#define LLSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int llsa_index_transpose_noalloc(const llsa_problem* prob, const int32_t* idx, int32_t* col_ptr, int32_t* perm,
                                 hipStream_t stream);

/*
 * llsa_attn_bwd -- gradients of the enriched sparse attention [LLSA review, "If this is right"
 * (backward over sparse indices only); abstract]: with Delta_t = dO_t . O_t and P = exp(z - lse),
 * dV_e += P dO_t, dS = P (dO_t . v_e - Delta_t), dQ_t += sigma dS k_e, dK_e += sigma dS q_t over each
 * query's entry set; gradients of pooled level-l tokens reach the raw tokens they pool with factor
 * B^-l.  No gradient flows through the Top-K choice or into pooled queries.  Key-side gradients are
 * gathered per key block through the CSC (no atomics).  bf16 only in this version (LLSA_ERR_DTYPE for
 * fp32).
 *   q, k, v, o, dout in: raw tensors (dtype); lse in: from llsa_attn_fwd; pk, pv (bf16 copies), idx: as
 *   forward (idx from llsa_select: any other idx is undefined behaviour);
 *   col_ptr, perm in: from llsa_index_transpose of the same idx.
 *   dq, dk, dv out: raw tensors (dtype).
 *   ws scratch of llsa_workspace_bytes(prob, LLSA_OP_ATTN_BWD) bytes (caller-owned).
 */
int llsa_attn_bwd(const llsa_problem* prob, const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, const void* pk, const void* pv, const int32_t* idx,
                  const int32_t* col_ptr, const int32_t* perm, void* dq, void* dk, void* dv, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* ---- host-only helpers (no GPU work) ---------------------------------------------------------- */

/* Validate `prob` and fill the defaults (levels, enrich_levels, scale) into `out`.  Returns a status. */
int llsa_resolve(const llsa_problem* prob, llsa_problem* out);
/* R = sum_{l=1..L} n / B^l (rows of one pyramid slice); < 0 on an invalid problem. */
int64_t llsa_pyramid_rows(const llsa_problem* prob);
/* sum_{l=1..T} (n/B^l + 1), T = max(1, L_e): col_ptr entries per batch*head; < 0 if invalid. */
int64_t llsa_colptr_len(const llsa_problem* prob);
/* sum_{l=1..T} (n/B^l) * K: perm entries per batch*head; < 0 if invalid. */
int64_t llsa_perm_len(const llsa_problem* prob);
/* Workspace bytes for `op` (LLSA_OP_*); O(n) per batch*head, never O(n^2).  0 for an invalid problem. */
size_t llsa_workspace_bytes(const llsa_problem* prob, int op);
/* Static, NUL-terminated description of a status code. */
const char* llsa_status_string(int status);

/* ---- streams ------------------------------------------------------------------------------------ */
/* Makes `waiter` wait, on the device, for the work enqueued on `signaler` so far, through an event with
 * no system-scope fence (HIP's hipEventDisableSystemFence): the results are visible to later kernels of
 * this device, not to the host or other devices.  For the two-stream step, in which the index transpose
 * runs beside the forward: one call after the selection (side waits for main) and one before the
 * backward (main waits for side).  Both streams belong to the current device; NULL is the default
 * stream.  The library creates and releases the event inside the call and keeps nothing.  Returns
 * LLSA_OK, or LLSA_ERR_LAUNCH if a HIP event call fails.
 * Stream capture: the calls of the path (pyramid, select, attn_fwd, index_transpose, attn_bwd) and this
 * one enqueue only kernels and event waits (no allocation, memset or host synchronisation), so a HIP
 * stream capture of the two-stream step replays with the results of the eager step.  The kernel timer
 * below records timing events and must stay disabled while a stream is captured. */
int llsa_stream_wait(hipStream_t waiter, hipStream_t signaler);

/* ---- kernel timing (for benchmarks) ------------------------------------------------------------ */
/* Kernel families of this library, for llsa_timing_read. */
enum {
  LLSA_KERNEL_POOL = 0,       /* pyramid pooling                                   */
  LLSA_KERNEL_SELECT = 1,     /* hierarchical Top-K, one launch per level          */
  LLSA_KERNEL_ATTN_FWD = 2,   /* enriched attention forward                        */
  LLSA_KERNEL_TRANSPOSE = 3,  /* CSR -> CSC: counts and scan, fill (or scatter, order) */
  LLSA_KERNEL_BWD_DQ = 4,     /* backward: dQ, Delta, pooled-token partials        */
  LLSA_KERNEL_BWD_REDUCE = 5, /* backward: pooled-token gradient reduction         */
  LLSA_KERNEL_BWD_DKDV = 6,   /* backward: dK, dV through the CSC                  */
  LLSA_KERNEL_SELECT_EXHAUSTIVE = 7, /* single-level exhaustive Top-K (not on the hot path) */
  LLSA_KERNEL_REORDER = 8,    /* 2-D-local index reordering                        */
  LLSA_KERNEL_COMPLEMENT = 9, /* complement lists of the complement reading        */
  LLSA_KERNEL_COUNT = 10
};
/* While enabled, every kernel this library launches is bracketed by two hipEvents recorded on its
 * launch stream (process-wide switch; off by default).  Enabling clears earlier records.  The events
 * are library-owned and released by the next llsa_timing_enable call.  Returns a status. */
int llsa_timing_enable(int on);
/* Waits for the recorded events of kernel family `kernel` and returns the summed duration (ms) and
 * the number of launches recorded since timing was enabled. */
int llsa_timing_read(int kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* LLSA_H */
