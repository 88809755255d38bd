/*
 * flashmask.h - C ABI of a gfx950 (MI355X) library for exact attention with a
 * column-wise sparse mask.
 *
 * Operation (FlashMask README, "Formulation"):
 *     O = softmax(Q K^T / sqrt(d) + M) V
 * with d the last dimension of Q and M the column-wise sparse mask of the
 * FlashMask README ("Overview") and the FlashMask-3 abstract: the mask is
 * indexed by key position and stores, per key column j, query-row interval
 * bounds. Four int32 vectors of length N describe it:
 *     row i is masked for column j  <=>  (causal && j > i)
 *                                     ||  LTS[j] <= i < LTE[j]
 *                                     ||  (!causal && UTS[j] <= i < UTE[j])
 * Intervals are half-open over 0-based rows; any int32 value is legal (a value
 * outside [0, N] acts as if clamped). Masked scores get zero probability. A
 * row whose keys are all masked outputs 0, has logsumexp -inf and contributes
 * no gradient. The dense mask never exists: mask memory is O(N) (FlashMask
 * abstract). Tiles the mask hides completely are skipped, tiles it does not
 * touch run without mask arithmetic, and only the rest test each element
 * (FlashMask README "Overview": sparsity is used to skip computation).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless stated otherwise. Tensors are
 *     contiguous row-major: Q, K [B, H, N, d]; V, O, dO [B, H, N, dv];
 *     logsumexp [B, H, N] float32; mask vectors [B, hm, N] int32 with
 *     hm == 1 (one mask shared by all heads) or hm == H (one per head).
 *   - lts == NULL: no lower interval (lte ignored). lte == NULL with lts set:
 *     LTE = N. Non-causal: uts and ute are both NULL (no upper interval) or
 *     both set; causal: uts/ute are ignored and may be NULL.
 *   - The caller owns all memory, including the workspace; the library never
 *     allocates, frees or synchronises. Every call only enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *     Results are valid once the caller has synchronised that stream.
 *   - Arguments are checked on the host before anything is enqueued. A failed
 *     check returns a status code and touches no output. A failed launch
 *     returns FM_ERROR_HIP. No exception crosses this interface and the
 *     library keeps no mutable global state beyond a per-device cache of
 *     the compute-unit count (read from the runtime; safe to call from
 *     several host threads at once).
 *   - B * H * N == 0 is a successful no-op. Offsets are 64-bit.
 *   - softmax_scale <= 0 or NaN selects 1/sqrt(d).
 *   - Supported (forward and backward): dtype FM_BF16 with d == dv in
 *     {64, 128, 256, 512} or d = 192 with dv = 128 (Q/K head dim larger than
 *     V's; README "News" and "Key Features": large head dims); FM_FP32 with
 *     d == dv in {64, 128, 256} or d = 192 with dv = 128. Others:
 *     FM_ERROR_NOT_SUPPORTED.
 */
#ifndef FLASHMASK_H
#define FLASHMASK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums are int-sized. C++ fixes int as their underlying type, so any
 * int a caller passes (an unknown status or dtype from C or a foreign-function
 * binding) is a valid value to test and reject; C gives them int
 * representation already. */
#ifdef __cplusplus
#define FM_ENUM_INT : int
#else
#define FM_ENUM_INT
#endif

typedef enum fm_status_e FM_ENUM_INT {
    FM_SUCCESS = 0,
    FM_ERROR_INVALID_VALUE = 1,       /* NULL required pointer, bad size, hm not in {1, H}, ... */
    FM_ERROR_NOT_SUPPORTED = 2,       /* (d, dv, dtype) combination not compiled in */
    FM_ERROR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < flashmask_workspace_size(...) */
    FM_ERROR_HIP = 4                  /* a kernel launch failed */
} fm_status_t;

typedef enum fm_dtype_e FM_ENUM_INT { FM_FP32 = 0, FM_BF16 = 1 } fm_dtype_t;

/* Static text for a status code; never NULL. */
const char* flashmask_status_string(fm_status_t status);

/* Column granularity Bt of the key-block table that flashmask_fwd and
 * flashmask_bwd accept as `kblock_minmax` (a table from
 * flashmask_tile_classify with block_k == flashmask_table_block()). */
int flashmask_table_block(void);

/* Tile shape (query rows x key columns) the forward (is_bwd == 0) or backward
 * (is_bwd != 0) kernel classifies and counts in `tile_counts`, for head dim d
 * and dtype. Returns FM_ERROR_NOT_SUPPORTED for a combination not compiled in. */
fm_status_t flashmask_tile_shape(int is_bwd, int d, fm_dtype_t dtype,
                                 int* block_q, int* block_k);

/* Bytes of device workspace flashmask_fwd (is_bwd == 0) or flashmask_bwd
 * (is_bwd != 0) needs for these sizes; 0 on invalid sizes (negative, hm not
 * in {1, H}, dims not supported, or sizes the kernels cannot address, which
 * flashmask_fwd/flashmask_bwd reject with FM_ERROR_NOT_SUPPORTED). The workspace
 * needs 256-byte alignment. It holds per-call state (the key-block table;
 * for the backward also delta, the base-2 logsumexp, the row sums of dS
 * the sink gradient uses and the work-queue counters of the dK/dV pass), so
 * calls that may run at the same time need separate workspaces. */
size_t flashmask_workspace_size(int is_bwd, int B, int H, int N, int d, int dv,
                                int hm, fm_dtype_t dtype);

/*
 * Key-block table and tile classes.
 *
 * kblock_minmax (out, int32 [B, hm, ceil(N/block_k), 8]): for every block of
 * block_k key columns [c0, c1), c1 = min(N, c0 + block_k), the min and max of
 * each vector in the order LTS min, LTS max, LTE min, LTE max, UTS min,
 * UTS max, UTE min, UTE max. Missing vectors take neutral values: no lower
 * interval -> LTS = LTE = N; lte NULL -> LTE = N; no upper interval (or
 * uts/ute NULL) -> UTS = UTE = 0. The table depends on the vectors only.
 *
 * tile_class (out, nullable, int8 [B, hm, ceil(N/block_q), ceil(N/block_k)]):
 * for rows [r0, r1) and columns [c0, c1), both clipped to N:
 *   0 (masked, skipped): (causal && c0 > r1 - 1) || (LTSmax <= r0 && LTEmin >= r1)
 *                        || (!causal && UTSmax <= r0 && UTEmin >= r1)
 *   2 (unmasked):        (!causal || c1 - 1 <= r0) && (LTEmax <= r0 || LTSmin >= r1)
 *                        && (causal || UTEmax <= r0 || UTSmin >= r1)
 *   1 (partial):         otherwise.
 * Conservative: a 0 or 2 is always exact, a 1 may be a tile without or with
 * only masked elements. The skipping rule follows the FlashMask README
 * ("Overview": mask sparsity skips unnecessary computation).
 *
 * block_q, block_k >= 1. Integer work: results are bit-exact.
 */
fm_status_t flashmask_tile_classify(const int32_t* lts, const int32_t* lte,
                                    const int32_t* uts, const int32_t* ute,
                                    int B, int hm, int N, int causal,
                                    int block_q, int block_k,
                                    int32_t* kblock_minmax, int8_t* tile_class,
                                    void* stream);

/*
 * Forward. q, k [B,H,N,d]; v [B,H,N,dv]; o (out) [B,H,N,dv] in dtype;
 * lse (out) [B,H,N] float32, natural log of sum_j exp(scale * q_i . k_j)
 * over open keys (-inf for a fully masked row). kblock_minmax (nullable): a
 * precomputed table at flashmask_table_block() granularity for these vectors
 * (reused across calls when the mask is fixed); NULL computes it in the
 * workspace. tile_counts (nullable, int64 [3], accumulated into, not
 * cleared): tiles of flashmask_tile_shape(0, ...) classified masked, partial
 * and unmasked. The output is bitwise deterministic.
 */
fm_status_t flashmask_fwd(const void* q, const void* k, const void* v,
                          const int32_t* lts, const int32_t* lte,
                          const int32_t* uts, const int32_t* ute, int hm,
                          const int32_t* kblock_minmax,
                          int B, int H, int N, int d, int dv, fm_dtype_t dtype,
                          int causal, float softmax_scale,
                          void* o, float* lse, int64_t* tile_counts,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward (FlashMask README "Overview": the library ships forward and
 * backward kernels; the gradient is the analytic one of the README
 * "Formulation" expression). Given o and lse from flashmask_fwd with the
 * same inputs and dout [B,H,N,dv], writes dq, dk [B,H,N,d] and dv_out
 * [B,H,N,dv] in dtype: the analytic gradient of O = softmax(scale Q K^T + M) V,
 *   dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 *   dK = scale dS^T Q.
 * tile_counts as in the forward, for flashmask_tile_shape(1, ...). All
 * three gradients are bitwise deterministic for both dtypes: dQ comes from a
 * query-major pass and dK, dV from a key-major pass, each summing in a fixed
 * order in registers (no atomics).
 */
fm_status_t flashmask_bwd(const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout,
                          const int32_t* lts, const int32_t* lte,
                          const int32_t* uts, const int32_t* ute, int hm,
                          const int32_t* kblock_minmax,
                          int B, int H, int N, int d, int dv, fm_dtype_t dtype,
                          int causal, float softmax_scale,
                          void* dq, void* dk, void* dv_out, int64_t* tile_counts,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Nq query rows against Nk keys (one context-parallel rank's share of the
 * rows: FlashMask-3 abstract), and an optional sink bias. Same contracts as
 * the entry points above with N split in two: Q, O, dO, dQ are [B,H,Nq,*], logsumexp [B,H,Nq]; K, V, dK,
 * dV are [B,H,Nk,*]; the mask vectors are [B,hm,Nk] and hold bounds on the Nq
 * rows (a missing lte means LTE = Nq; the causal test is j > i). The table is
 * [B,hm,ceil(Nk/block_k),8] and the class map [B,hm,ceil(Nq/block_q),
 * ceil(Nk/block_k)]. Nk == 0 gives O = 0, LSE = -inf, dQ = 0; Nq == 0 gives
 * dK = dV = 0. The entry points above are these with Nq = Nk = N.
 */
size_t flashmask_workspace_size_qk(int is_bwd, int B, int H, int Nq, int Nk, int d, int dv,
                                   int hm, fm_dtype_t dtype);

fm_status_t flashmask_tile_classify_qk(const int32_t* lts, const int32_t* lte,
                                       const int32_t* uts, const int32_t* ute,
                                       int B, int hm, int Nq, int Nk, int causal,
                                       int block_q, int block_k,
                                       int32_t* kblock_minmax, int8_t* tile_class,
                                       void* stream);

/*
 * sink (nullable, float32 [H], device): sink bias (README "News" names it;
 * the reading taken here): per head h a logit s_h, in the units of the
 * scaled scores, joins every row's softmax as one more always-open entry
 * whose value vector is zero:
 *     LSE_i = log(exp(s_h) + sum_{open j} exp(scale q_i . k_j)),
 *     O_i = sum_{open j} exp(scale q_i . k_j - LSE_i) v_j.
 * A row with nothing open gets O = 0 and LSE = s_h. The backward must get
 * the same sink (the saved LSE includes it); dsink (nullable, float32 [H],
 * device, written only when sink is given) receives
 *     d loss / d s_h = -sum_{b, i} exp(s_h - LSE_i) (dO_i . O_i),
 * reduced in a fixed order (deterministic).
 */
fm_status_t flashmask_fwd_qk(const void* q, const void* k, const void* v,
                             const int32_t* lts, const int32_t* lte,
                             const int32_t* uts, const int32_t* ute, int hm,
                             const int32_t* kblock_minmax,
                             int B, int H, int Nq, int Nk, int d, int dv, fm_dtype_t dtype,
                             int causal, float softmax_scale, const float* sink,
                             void* o, float* lse, int64_t* tile_counts,
                             void* workspace, size_t workspace_bytes, void* stream);

fm_status_t flashmask_bwd_qk(const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout,
                             const int32_t* lts, const int32_t* lte,
                             const int32_t* uts, const int32_t* ute, int hm,
                             const int32_t* kblock_minmax,
                             int B, int H, int Nq, int Nk, int d, int dv, fm_dtype_t dtype,
                             int causal, float softmax_scale, const float* sink,
                             void* dq, void* dk, void* dv_out, float* dsink,
                             int64_t* tile_counts,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward that allocates nothing and takes no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments and
 * results as flashmask_bwd_qk without `workspace` / `workspace_bytes`: the
 * workspace is a static device array of FLASHMASK_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends (its address
 * is looked up once per device on the first call). A problem whose
 * flashmask_workspace_size_qk(1, ...) exceeds that returns
 * FM_ERROR_WORKSPACE_TOO_SMALL before anything is enqueued (16 MiB holds
 * B * H * Nq up to about 1.3 million query rows). The array keeps the last
 * call's contents; every call writes what it reads before reading it (the
 * work-queue counters are reset by the call's own first kernel, no memset).
 * All calls on one GPU share the array: calls that may overlap on one GPU
 * (on different streams, or from several host threads) race and must be
 * serialised by the caller.
 */
#define FLASHMASK_NOALLOC_SCRATCH_BYTES (16u << 20)

fm_status_t flashmask_bwd_noalloc(const void* q, const void* k, const void* v,
                                  const void* o, const float* lse, const void* dout,
                                  const int32_t* lts, const int32_t* lte,
                                  const int32_t* uts, const int32_t* ute, int hm,
                                  const int32_t* kblock_minmax,
                                  int B, int H, int Nq, int Nk, int d, int dv, fm_dtype_t dtype,
                                  int causal, float softmax_scale, const float* sink,
                                  void* dq, void* dk, void* dv_out, float* dsink,
                                  int64_t* tile_counts, void* stream);

/* Largest nchunks flashmask_localize accepts. */
int flashmask_max_chunks(void);

/*
 * Localise the mask to one rank's query rows (FlashMask-3 abstract: each rank
 * localises the column-wise mask without communication). The rank holds the
 * global rows of `nchunks` chunks [chunks[2c], chunks[2c+1]) (HOST pointer,
 * int32 pairs; sorted, disjoint, non-empty, inside [0, n_rows]; at most
 * flashmask_max_chunks()), in that order as its local rows 0..Nq-1. Input:
 * the global vectors [B,hm,Nk] (same NULL conventions as above, bounds on
 * n_rows global rows). Output (device, [B,hm,Nk] each, all four written):
 * the vectors of the same mask restricted to the local rows, non-causal:
 *     local(t) = sum_c clamp(t - q0_c, 0, q1_c - q0_c)
 *     LTS', LTE' = local(LTS), local(LTE)  (no lower interval: Nq, Nq)
 *     causal:     UTS', UTE' = 0, local(j)
 *     non-causal: UTS', UTE' = local(UTS), local(UTE)  (none: 0, 0)
 * Integer work: bit-exact. Pass the outputs with causal = 0 and the rank's
 * Q rows (Nq = total chunk length) to flashmask_fwd_qk / flashmask_bwd_qk.
 */
fm_status_t flashmask_localize(const int32_t* lts, const int32_t* lte,
                               const int32_t* uts, const int32_t* ute,
                               int B, int hm, int Nk, int n_rows, int causal,
                               const int32_t* chunks, int nchunks,
                               int32_t* lts_out, int32_t* lte_out,
                               int32_t* uts_out, int32_t* ute_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHMASK_H */
