/*
 * mlora: multi-LoRA adapted linear layer for AMD Instinct MI355X (gfx950).
 *
 * Computes, for a batch of T tokens in which every token carries its own K adapter slots,
 *
 *   y[t] = W x[t] + sum_{j : a = idx[t][j] != -1}  s[t][j] * f[a] * B[a] (A[a] x[t])
 *
 * with f[a] = alpha_a / r_a, or alpha_a / sqrt(r_a) for rsLoRA adapters.
 *
 * Sources (web pages):
 *  - "Multi-LoRA Serving Explained" (sevydevy.com): the LoRA layer W x + B(A x) scaled by
 *    alpha/r (B is out x rank, A is rank x in); one shared base product for the whole batch plus
 *    a per-token side path found through the token's slot id, -1 meaning base model only (the
 *    six-token batching script); stacked zero-padded slot buffers of width max_lora_rank
 *    (section "Why max-lora-rank costs memory even for small adapters"); sorting tokens by slot
 *    before shrink/expand and skipping the LoRA kernels when no token uses an adapter.
 *  - "[RFC]: Per-request activation of multiple LoRA adapters with static scales" (vLLM issue
 *    51940), Proposed Change: k slots per token with sentinel fill, per-adapter static scales,
 *    the slots iterated inside the kernels.
 *  - vLLM learning book, chapter "04. LoRA Serving", section 6 (PunicaWrapper): add_lora_linear,
 *    add_shrink (scaled x A, rank-wide intermediate) and add_expand (y += intermediate B).
 *  - "[vLLM] LoRA" (blog.secrett2633.cloud), PEFTHelper section: the rsLoRA factor.
 *
 * Conventions shared by every entry point:
 *  - Device pointers unless marked "host".  bf16 buffers are passed as void* holding bfloat16
 *    bits.  Everything is row-major and contiguous; base pointers must be 16-byte aligned.
 *  - The caller owns every buffer.  The library allocates no device memory on these calls:
 *    scratch space comes in through (ws, ws_bytes), sized by mlora_workspace_size(); its
 *    contents need no preparation and carry nothing from one call to the next.
 *  - Calls enqueue work on `stream` and return; the status reports only the synchronous
 *    argument checks and launch errors (MLORA_ERR_HIP).  No exception crosses the ABI.
 *  - Calls on one stream are ordered; two calls that share a workspace must not overlap.
 *  - Indices outside [-1, S) are undefined behaviour on the fast path; mlora_validate() checks
 *    them (and the ranks) synchronously.
 *  - Results are deterministic: the same inputs give the same output bits on every run.
 */
#ifndef MLORA_H
#define MLORA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLORA_OK = 0,
    MLORA_ERR_ARG = 1,         /* null pointer, negative size, misaligned pointer            */
    MLORA_ERR_SHAPE = 2,       /* inconsistent sizes (slice table, n_in not a multiple of 8) */
    MLORA_ERR_RANK = 3,        /* an adapter rank outside [1, R]                             */
    MLORA_ERR_INDEX = 4,       /* a slot index outside [-1, S)                               */
    MLORA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than mlora_workspace_size()   */
    MLORA_ERR_HIP = 6,         /* a HIP call or kernel launch failed                         */
    MLORA_ERR_UNSUPPORTED = 7  /* outside the supported limits below                         */
} mlora_status;

/* Supported limits. */
#define MLORA_MAX_SLICES 4        /* output slices of a merged layer (QKV = 3)                 */
#define MLORA_MAX_RANK 512        /* slot width R: a power of two from 8 to 512                */
#define MLORA_MAX_SLOTS 16384     /* S                                                         */
#define MLORA_MAX_K 8             /* adapter slots per token                                   */

/* flags of mlora_linear */
#define MLORA_NO_ADAPTERS 1u      /* host hint: no token uses an adapter; run the base only    */
#define MLORA_PATH_DECODE 2u      /* force the decode kernels (token chunks of 64)             */
#define MLORA_PATH_TILED 4u       /* force the tiled prefill kernels (256-token tiles)         */
#define MLORA_W_PACKED 8u         /* W is in the packed layout of mlora_pack_weight            */
#define MLORA_PATH_GROUPED 16u    /* force the grouped decode: decode base, LoRA per adapter   */

/*
 * The adapter slot set of ONE layer: S slots, each R wide (R = max_lora_rank), an adapter of
 * rank r < R sitting zero-padded in the first r rows of A and first r columns of B.
 * A merged layer (e.g. QKV) has n_slices output slices: slice s owns output rows
 * [slice_start[s], slice_start[s+1]) and has its own down matrix A[a][s].
 */
typedef struct {
    const void *A;          /* bf16 [S][n_slices][R][n_in]; rows >= rank[a] must be zero     */
    const void *B;          /* bf16 [S][n_out][R];          cols >= rank[a] must be zero     */
    const float *factor;    /* fp32 [S]: alpha/r or alpha/sqrt(r) (see mlora_factor)         */
    int32_t S;              /* number of slots, 1..MLORA_MAX_SLOTS                           */
    int32_t R;              /* slot width, a power of two, 8 <= R <= MLORA_MAX_RANK          */
    int32_t n_slices;       /* 1..MLORA_MAX_SLICES                                           */
    int32_t slice_start[MLORA_MAX_SLICES + 1]; /* host values: 0 = s_0 < s_1 < .. = n_out.
                                                  With n_slices == 1 it may be all zero,
                                                  meaning {0, n_out}.                        */
    const int32_t *rank;    /* int32 [S] device: each slot's true rank r <= R, or NULL (= R).
                               With it the kernels skip the zero padding beyond r (same
                               results: the skipped products are exact zeros).  Values must be
                               in [1, R] (mlora_validate); larger ones are read as R.        */
} mlora_slots;

/* Text for a status code (static storage). */
const char *mlora_status_string(mlora_status status);

/* Text of the last HIP failure seen by this thread (the call that failed and HIP's message),
 * or "" if none; valid until the next failing call on the same thread. */
const char *mlora_last_error(void);

/*
 * Host helper: the scale factor of one adapter, alpha/r, or alpha/sqrt(r) when use_rslora is
 * non-zero ("[vLLM] LoRA", PEFTHelper section).  r is the adapter's true rank, not R.
 * Computed in double and rounded once to float.  Returns NaN for r < 1.
 */
float mlora_factor(float alpha, int32_t r, int32_t use_rslora);

/*
 * Host helper: bytes of one layer's slot buffers, S * (n_slices*R*n_in + n_out*R) * 2
 * ("Multi-LoRA Serving Explained", memory script: rank x (in + out) 16-bit numbers per adapted
 * layer, slots sized at max_lora_rank).  Returns -1 on negative arguments.
 */
int64_t mlora_slot_bytes(int32_t S, int32_t R, int64_t n_in, int64_t n_out, int32_t n_slices);

/*
 * Bytes of workspace that mlora_plan / mlora_shrink / mlora_linear need for these sizes
 * (an upper bound over every index map of this shape).  Returns 0 on invalid arguments.
 * The largest part is the tiled path's V blocks, about T x n_slices x 4 R x min(256 K, S)
 * bytes (T up to 1,048,576 tokens a launch): each 256-token tile's block is sized for a tile
 * that holds min(256 K, S) adapters, since a tile with too many adapters for the extra
 * k-steps takes the per-adapter route only while its fp32 sums fit the 64 MiB kept for them
 * (else the extra k-steps).  The rest: at most 64 MiB each of those fp32 sums and of the
 * shrink's partial blocks, and the decode kernels' split partials (16 n_out bytes a token of a
 * launch of up to 512).  For example 605 MiB at T = 16384, 4096 -> 11008, S = 100, R = 64;
 * 36 MiB for the 64-token decode batch at 4096 -> 4096; 3.2 GiB for a merged QKV layer with
 * S = 1000, R = 64 at T = 16384 (the size is linear in T: such callers can split the batch).
 */
size_t mlora_workspace_size(int64_t T, int32_t K, int64_t n_in, int64_t n_out,
                            const mlora_slots *slots);

/*
 * Slot activation ("Multi-LoRA Serving Explained": slots sized for max_lora_rank R, an adapter
 * of rank r < R zero-padded in its slot; an adapter whose rank exceeds R is rejected).  Loads
 * one adapter into slot `slot` of a slot set whose device buffers are A, B and factor (the
 * same buffers and layout as mlora_slots: A bf16 [S][n_slices][R][n_in], B bf16 [S][n_out][R],
 * factor fp32 [S]):
 *   A_src  bf16 [n_slices][r][n_in]   the adapter's down matrices (host or device memory)
 *   B_src  bf16 [n_out][r]            its up matrix (host or device memory)
 *   r      its true rank, 1 <= r <= R, else MLORA_ERR_RANK
 *   f      its scale factor (mlora_factor), written to factor[slot]
 * Rows r..R-1 of the slot's A and columns r..R-1 of its B are set to zero.  Everything is
 * enqueued on `stream` (asynchronous copies, then one kernel; no memset): host sources must
 * stay valid until the stream reaches the call, and are copied asynchronously only when
 * pinned.  The slot must not be in use by work in flight on other streams.  MLORA_ERR_ARG on
 * a NULL pointer, slot outside [0, S) or sizes below 1; MLORA_ERR_UNSUPPORTED outside the
 * limits above (S, R, n_slices).
 */
mlora_status mlora_slot_load(void *A, void *B, float *factor, int32_t S, int32_t R,
                             int32_t n_slices, int64_t n_in, int64_t n_out, int32_t slot,
                             const void *A_src, const void *B_src, int32_t r, float f,
                             hipStream_t stream);

/*
 * Packed base weight (a relayout for the matrix cores, done once when a weight is loaded; not
 * from the pages): the layer's W bf16 [n_out][n_in] rearranged so that each 16-row x 32-column
 * block is 1 KB contiguous in the order the v_mfma_f32_16x16x32_bf16 A operand takes it
 * (lane l: row l % 16, columns 8 (l / 16) .. +8), blocks ordered by row group, then column
 * block; zero padded to 16 rows and 32 columns:
 *   Wp[rg][kb][l][e] = W[16 rg + l % 16][32 kb + 8 (l / 16) + e]
 * mlora_packed_weight_bytes returns its size (0 on invalid sizes); mlora_pack_weight writes it
 * (one kernel on `stream`; W and Wp device, 16-byte aligned, not overlapping).  mlora_linear
 * with MLORA_W_PACKED then takes Wp in place of W and gives the same output bits: the
 * kernels read whole cache lines of W per load instruction.  MLORA_ERR_ARG on NULL or
 * misaligned pointers or sizes below 1, MLORA_ERR_SHAPE if n_in is not a multiple of 8.
 */
int64_t mlora_packed_weight_bytes(int64_t n_out, int64_t n_in);
mlora_status mlora_pack_weight(const void *W, int64_t n_out, int64_t n_in, void *Wp,
                               hipStream_t stream);

/*
 * Synchronous check of an index map and of the adapter ranks (blocks on `stream`).
 *   idx   int32 [T][K] device
 *   rank  int32 [S] host, true adapter ranks (may be NULL to skip the rank check)
 * Returns MLORA_ERR_INDEX if some idx is outside [-1, S), MLORA_ERR_RANK if some rank is
 * outside [1, R] ("Multi-LoRA Serving Explained": an adapter whose rank exceeds max_lora_rank
 * is rejected); the offending value is written to *bad_value (may be NULL).
 */
mlora_status mlora_validate(const int32_t *idx, int64_t T, int32_t K, const mlora_slots *slots,
                            const int32_t *rank, int64_t *bad_value, hipStream_t stream);

/*
 * Token-mapping plan ("Multi-LoRA Serving Explained": tokens sorted by slot, one group per
 * adapter; six-token script's stable argsort).  The flat pairs p = t*K + j are sorted by slot
 * idx[p] ascending, ties in ascending p; pairs holding -1 are dropped.
 * Outputs (device):
 *   perm       int32 [T*K]  first n_pairs entries: sorted pair indices
 *   seg_slot   int32 [S]    first n_seg entries: slot of each segment, ascending
 *   seg_start  int32 [S]    first position of the segment in perm
 *   seg_len    int32 [S]    its length
 *   counts     int32 [2]    {n_seg, n_pairs}
 * Exactly one result is correct, so the outputs are bit-exact.  T = 0 writes counts {0, 0}.
 * ws: at least the plan's part of mlora_workspace_size for T, K and S (MLORA_ERR_WORKSPACE
 * otherwise; maps of up to 8192 pairs over up to 1000 slots are sorted in one launch that
 * leaves it untouched).
 */
mlora_status mlora_plan(const int32_t *idx, int64_t T, int32_t K, int32_t S, int32_t *perm,
                        int32_t *seg_slot, int32_t *seg_start, int32_t *seg_len,
                        int32_t *counts, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Shrink (learning book section 6, add_shrink; RFC stage 4: the K slots in one pass):
 *   v[j][t][s*R + rho] = scale[t][j] * factor[a] * sum_i A[a][s][rho][i] x[t][i],  a = idx[t][j]
 * and v[j][t][:] = 0 where idx[t][j] == -1.
 *   x      bf16 [T][n_in]
 *   idx    int32 [T][K]
 *   scale  fp32 [T][K], or NULL for all ones
 *   v      fp32 [K][T][n_slices*R]   (output, overwritten)
 */
mlora_status mlora_shrink(const void *x, int64_t T, int64_t n_in, const mlora_slots *slots,
                          const int32_t *idx, int32_t K, const float *scale, float *v, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/*
 * Expand (learning book section 6, add_expand):
 *   y[t][n] = bf16( y[t][n] + sum_j [idx[t][j] != -1] sum_rho B[a][n][rho] v[j][t][s(n)*R+rho] )
 * where s(n) is the slice owning row n.  Rows whose slots are all -1 are left untouched.
 *   v  fp32 [K][T][n_slices*R]   (as written by mlora_shrink)
 *   y  bf16 [T][n_out]           (in/out; one rounding of the sum)
 */
mlora_status mlora_expand(const float *v, int64_t T, int64_t n_out, const mlora_slots *slots,
                          const int32_t *idx, int32_t K, void *y, hipStream_t stream);

/*
 * The whole layer, one rounding of each output:
 *   y[t] = bf16( W x[t] + sum_j [idx[t][j] != -1] scale[t][j] factor[a] B[a] (A[a] x[t]) )
 *   x  bf16 [T][n_in];  W  bf16 [n_out][n_in] (row n is output n);  y  bf16 [T][n_out] (out)
 *   idx, scale as in mlora_shrink.  slots may be NULL only with MLORA_NO_ADAPTERS.
 * With flags & MLORA_NO_ADAPTERS no LoRA kernel is launched (y = bf16(W x)); without it, an
 * all-sentinel map gives the same values.  T = 0 is a no-op.  By default the library picks
 * the decode kernels or the tiled kernels, whichever a host-side model of their measured
 * rates estimates faster for the sizes (the tiled kernels from about 1536 tokens at 4096 ->
 * 4096, 768 at 4096 -> 11008, 256 at vocabulary-wide outputs).  Where the decode kernels
 * are picked, a batch of 128 or more tokens whose per-token adapter reads (each (token, slot)
 * pair's A rows and B columns) would exceed both four times W's bytes and 200 MB
 * takes the grouped decode ("Multi-LoRA Serving Explained", the segmented method: tokens
 * sorted by adapter so that each adapter is read once per group): the decode kernels' base
 * product, the LoRA terms computed per adapter over its tokens.  The decode kernels compute
 * the shrink inside the GEMM pass, or, where 64 output rows would get 4 or more (token, slot)
 * pairs of a 64-token chunk (narrow outputs), with the per-pair shrink kernel ahead of a GEMM
 * of the base alone.  MLORA_PATH_DECODE /
 * MLORA_PATH_TILED / MLORA_PATH_GROUPED force one (more than one set: MLORA_ERR_ARG;
 * MLORA_PATH_GROUPED where the fp32 sums of one launch's up to 512 tokens exceed what the
 * grouped expand keeps, 64 MiB or one 256-token tile: MLORA_ERR_UNSUPPORTED).
 * mlora_workspace_size() covers every path.  With
 * MLORA_W_PACKED, W points to the packed layout written by mlora_pack_weight (same output
 * bits).
 */
mlora_status mlora_linear(const void *x, const void *W, int64_t T, int64_t n_in, int64_t n_out,
                          const mlora_slots *slots, const int32_t *idx, int32_t K,
                          const float *scale, void *y, uint32_t flags, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Which kernels mlora_linear runs for these sizes, slots and flags: MLORA_PATH_DECODE,
 * MLORA_PATH_TILED or MLORA_PATH_GROUPED (the choice is made on the host from the shapes and
 * flags alone, as described above; idx is not read).  Host only, no GPU call; slots' data
 * pointers are not checked.  Returns 0 where mlora_linear would fail its checks on these
 * arguments (sizes, slot geometry, conflicting flags, MLORA_PATH_GROUPED that does not fit).
 */
uint32_t mlora_linear_path(int64_t T, int64_t n_in, int64_t n_out, const mlora_slots *slots,
                           int32_t K, uint32_t flags);

/*
 * mlora_linear for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * output bits as mlora_linear with the same arguments, but its scratch space is a fixed array
 * of MLORA_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the process ends)
 * instead of a caller-provided workspace.  The caller still passes inputs and outputs.  It
 * calls no hipMalloc, hipFree or allocating routine.  A call whose path needs more scratch than
 * the fixed size (e.g. large tiled batches, very wide outputs) returns MLORA_ERR_WORKSPACE
 * before launching anything, with the needed size in mlora_last_error().  All calls on one GPU
 * share its array: calls that may overlap on one GPU (other streams, other threads) race and
 * must not be issued.  The array belongs to the device of `stream` (the current device for the
 * null stream).
 */
#define MLORA_NOALLOC_SCRATCH_BYTES (64u << 20)
mlora_status mlora_linear_noalloc(const void *x, const void *W, int64_t T, int64_t n_in,
                                  int64_t n_out, const mlora_slots *slots, const int32_t *idx,
                                  int32_t K, const float *scale, void *y, uint32_t flags,
                                  hipStream_t stream);

/*
 * Profiling hook (not part of the computation).  mlora_trace_start creates 2*capacity HIP
 * events (no device memory); from then on every mlora_linear call records one event on its
 * stream right before and one right after each launch of its main product kernel (the decode
 * GEMM or the tiled GEMM), every mlora_shrink / mlora_expand call around its one kernel, and
 * every mlora_plan call around its kernels (one duration for the one or three), for the first
 * `capacity` launches.
 * mlora_trace_stop waits for the recorded events, writes the duration of launch i in
 * milliseconds to ms[i] (host array of `capacity` floats; NULL discards them), releases the
 * events and returns the number of durations written (-1 on a HIP error).
 * Process-wide state, guarded by a lock; start returns MLORA_ERR_ARG unless
 * 1 <= capacity <= 2^20 and MLORA_ERR_HIP if an event cannot be created.
 */
mlora_status mlora_trace_start(int32_t capacity);
int32_t mlora_trace_stop(float *ms, int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* MLORA_H */
