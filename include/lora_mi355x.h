/*
 * lora_mi355x.h -- C ABI of the MI355X (gfx950) multi-adapter LoRA projection library.
 *
 * Operations (pages as titled):
 *   - lora_shrink / lora_expand: the chunked-SGMV LoRA shrink and expand of "Decode LoRA kernels
 *     are optimized" (sgl-kernel-xpu pull request 550), Summary: a gathered grouped GEMM (rows of
 *     x read through a token permutation, one rank block per output slice) and a scattered grouped
 *     GEMM whose epilogue applies the adapter scaling and the per-slice column offsets, driven by
 *     seg_indptr / weight_indices / permutation / slice offsets. The weight operand is stored
 *     [out][in] row-major, as in the masked operand load shown in that page's review thread.
 *   - lora_mlp_fused_train / lora_mlp_prepare_backward / lora_mlp_backward: the training
 *     forward (storing the gate and up pre-activations) and the gradients of the same MLP.
 *   - lora_mlp_fused: the single-adapter LoRA MLP with fused SwiGLU of "Add optional fast lora
 *     path for qwen2/qwen3 on npu" (ms-swift pull request 9754), What this PR does and
 *     Compatibility checks (dropout 0, one adapter, no bias, unmerged weights).
 *   - lora_linear_fused / lora_qkv_fused: the single-adapter LoRA attention projections (output,
 *     and query/key/value of one x) of the same fast path (pull request 9754).
 *   - lora_embedding_a: the embedding LoRA-A product of the same LoRA op family (pull request
 *     550), sized without a longest-segment bound.
 *   - lora_schedule_tiles: export of the device segment schedule (the on-device segment scheduler
 *     named in the Summary of pull request 550) for checking.
 *   - lora_check_metadata: the value checks that pull request 550 (Behaviour changes) moves out of
 *     the default path; here they are an explicit, synchronizing call.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory (hipMalloc or torch CUDA
 *     tensors) of the current HIP device; host pointers are named as such.
 *   - The caller owns every buffer. No entry point allocates, frees or keeps device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *     without waiting, except lora_check_metadata, which waits for its own result.
 *   - No entry point throws or aborts. Argument errors are reported before anything is enqueued
 *     and leave every output untouched.
 *   - Metadata values (seg_indptr, weight_indices, permutation, lora_ranks, slice_offsets) are not
 *     checked by the compute calls: values outside the rules of lora_check_metadata give
 *     undefined results (wrong output or a GPU memory fault), as pull request 550 specifies.
 *   - Element strides (ld*) are in elements, not bytes. 16-byte aligned pointers and strides that
 *     keep every row 16-byte aligned take the vector-load path; any other alignment is accepted
 *     and takes narrower loads.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_EINVAL = 1,        /* a null pointer with a nonzero extent, bad sizes or strides */
  LORA_EUNSUPPORTED = 2,  /* dtype or size outside what the kernels implement */
  LORA_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace_size query */
  LORA_EHIP = 4,          /* the HIP runtime reported an error while enqueuing */
  LORA_EVALUE = 5         /* lora_check_metadata found invalid metadata */
} lora_status;

typedef enum lora_dtype {
  LORA_F32 = 0,   /* IEEE binary32 */
  LORA_BF16 = 1,  /* bfloat16 */
  LORA_F16 = 2    /* IEEE binary16 */
} lora_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* lora_status_str(lora_status s);

/* Library version string, e.g. "lora_mi355x 0.1 gfx950". */
const char* lora_version(void);

/*
 * lora_shrink -- h = x[perm] * A_a^T per segment, one rank block per slice.
 *
 * For segment g (sorted positions seg_indptr[g] .. seg_indptr[g+1]-1), adapter
 * a = weight_indices[g], rank r = lora_ranks[a], every sorted position i in the segment, slice
 * s < S and j < R:
 *     h[i][s*R + j] = round( sum_{k<K} x[permutation[i]][k] * A[a][s*R + j][k] )   for j < r
 *     h[i][s*R + j] = 0                                                             for j >= r
 * accumulated in fp32 and rounded once (round to nearest even) to `dtype`.
 *
 *   dtype          element type of x, w_a and h.
 *   T              tokens (rows of x and of h); T == 0 is a no-op.
 *   K              input features (columns read from each x / A row), K >= 1.
 *   S, R           slices and padded rank; 1 <= S, 1 <= R, S*R <= 512.
 *   L              adapters stacked in w_a.
 *   G              segments; G == 0 is a no-op.
 *   x              device [T][ldx], ldx >= K; row t is token t. Only the first K entries of a row
 *                  are read.
 *   w_a            device [L*S*R][lda], lda >= K: row (a*S + s)*R + j holds A[a][s*R+j][:].
 *                  Rows with j >= lora_ranks[a] are never read.
 *   seg_indptr     device int32 [G+1]: 0 = seg_indptr[0] <= ... <= seg_indptr[G] = T.
 *   weight_indices device int32 [G], values in [0, L).
 *   permutation    device int32 [T], a bijection of [0, T): sorted position i reads token row
 *                  permutation[i]; NULL means the identity (tokens already grouped by segment:
 *                  the non-chunked LoRA-A product of the prefill path).
 *   lora_ranks     device int32 [L], values in [0, R].
 *   h              device [T][ldh], ldh >= S*R; row i is sorted position i. Columns >= S*R are
 *                  not written.
 *   workspace      device scratch of at least lora_shrink_workspace_size(...) bytes, 16-byte
 *                  aligned; may be NULL when that size is 0. When the size is nonzero its first
 *                  32 KiB are arrival counters that MUST hold zeros before the first call that
 *                  uses the workspace (zero it once, e.g. with hipMemset, when allocating it);
 *                  every call leaves them zero again, so a workspace can be reused across calls
 *                  and in captured graphs with no clearing. The rest holds the segment schedule
 *                  for many segments and the fp32 partial sums of the split reduction: when one
 *                  workgroup per tile would leave compute units idle, the (tile, K step) work is
 *                  shared out evenly over about one workgroup per compute unit, and the last
 *                  workgroup to finish a piece of a tile adds the tile's pieces in a fixed order
 *                  (results do not depend on timing). Calls that overlap in time (different
 *                  streams) must not share a workspace. Its other contents are undefined after
 *                  the call.
 */
lora_status lora_shrink(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t L,
                        int32_t G, const void* x, int64_t ldx, const void* w_a, int64_t lda,
                        const int32_t* seg_indptr, const int32_t* weight_indices,
                        const int32_t* permutation, const int32_t* lora_ranks, void* h, int64_t ldh,
                        void* workspace, size_t workspace_bytes, void* stream);

size_t lora_shrink_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                  int32_t G);

/*
 * lora_shrink_noalloc -- lora_shrink for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same operation,
 * arguments, kernels and results as lora_shrink, with no workspace argument. Its scratch (segment
 * schedule, partial sums, arrival counters) is a fixed array of
 * lora_shrink_noalloc_max_workspace() bytes (16 MiB) in the library's own device memory, one per
 * GPU, held until the process ends; its address is looked up once per device, on that device's
 * first call. The call allocates and frees nothing. It returns LORA_EWORKSPACE when the problem
 * needs more scratch than that (lora_shrink_workspace_size above 16 MiB), other errors as
 * lora_shrink. Every call on one GPU shares that GPU's array and leaves its contents there; the
 * counters a call uses are cleared at its start by a small fill kernel on `stream` (no memset), so
 * the call can be captured in a graph. Calls that can overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race on the array and give undefined results: order
 * them on one stream. `stream` must belong to the current device.
 */
lora_status lora_shrink_noalloc(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                int32_t L, int32_t G, const void* x, int64_t ldx,
                                const void* w_a, int64_t lda, const int32_t* seg_indptr,
                                const int32_t* weight_indices, const int32_t* permutation,
                                const int32_t* lora_ranks, void* h, int64_t ldh, void* stream);

size_t lora_shrink_noalloc_max_workspace(void);

/*
 * lora_plan -- an explicit choice of kernel shape for lora_shrink_ex / lora_expand_ex, for
 * measurement sweeps and for tests that reach every shape. Every field -1 (or a NULL plan) is
 * the library's own choice, which is what lora_shrink / lora_expand make. A plan is an input of
 * the one call: the library keeps no state between calls. Results are identical for every plan
 * up to the fp32 summation order. A field outside its range makes the call return LORA_EINVAL
 * (and the workspace query 0).
 *   shrink_kernel   0 operands loaded straight into MFMA registers; 1 staged through LDS; 2 the
 *                   wave-reduction (GEMV) form: packed dot products and cross-lane sums instead
 *                   of MFMA, one workgroup per 16-token tile and 16-column block (split ignored).
 *                   1 and 2 are taken only for 16-bit types with 16-byte aligned x and A rows
 *                   and K % 8 == 0, else 0 runs.
 *   shrink_shape    shape of the chosen kernel: 0 .. LORA_SHRINK_RING_SHAPES - 1 (kernel 0) or
 *                   0 .. LORA_SHRINK_LDS_SHAPES - 1 (kernel 1).
 *   shrink_split    0: one workgroup per tile over all of K; n in 1 .. 65535: n workgroups share
 *                   the (tile, K step) work evenly.
 *   shrink_finish   with a split: 1 the last workgroup of each tile adds the pieces in the same
 *                   launch (arrival counters in the workspace); 0 a second launch adds them.
 *   expand_shape    0 .. LORA_EXPAND_SHAPES - 1; shapes 8 and 9 need 16-bit types, padded rank
 *                   16 and 16-byte aligned h, B and y rows (otherwise shape 6 runs).
 *   expand_block_n  columns per expand workgroup, 1 .. 65536 (rounded up to the shape's unit).
 */
typedef struct lora_plan {
  int32_t shrink_kernel;
  int32_t shrink_shape;
  int32_t shrink_split;
  int32_t shrink_finish;
  int32_t expand_shape;
  int32_t expand_block_n;
} lora_plan;

#define LORA_SHRINK_RING_SHAPES 5
#define LORA_SHRINK_LDS_SHAPES 13
#define LORA_EXPAND_SHAPES 10

/* lora_shrink with an explicit plan (NULL: as lora_shrink); the workspace query must be made
 * with the same plan. */
lora_status lora_shrink_ex(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                           int32_t L, int32_t G, const void* x, int64_t ldx, const void* w_a,
                           int64_t lda, const int32_t* seg_indptr, const int32_t* weight_indices,
                           const int32_t* permutation, const int32_t* lora_ranks, void* h,
                           int64_t ldh, const lora_plan* plan, void* workspace,
                           size_t workspace_bytes, void* stream);

size_t lora_shrink_workspace_size_ex(lora_dtype dtype, int64_t T, int64_t K, int32_t S,
                                     int32_t R, int32_t G, const lora_plan* plan);

/*
 * lora_expand -- y[perm[i]][slice s] += scale_a * h_i,s * B_a^T (scaled scatter-add).
 *
 * For segment g (adapter a, rank r, scale = scalings[a]), sorted position i in it, slice s and
 * output column n with slice_offsets[s] <= n < slice_offsets[s+1]:
 *     y[permutation[i]][n] = round( y[permutation[i]][n]
 *                                   + scale * sum_{j<r} h[i][s*R + j] * B[a][n][j] )
 * with an fp32 accumulation and one rounding to `dtype` per stored element. Entries of y outside
 * the slices, and every row of a rank-0 adapter, are neither read nor written.
 *
 *   T, S, L, G     as for lora_shrink; permutation as for lora_shrink (NULL: identity, the
 *                  non-chunked LoRA-B product of the prefill path).
 *   R              padded rank, 1 <= R <= 64 (bf16, fp16) or 32 (fp32).
 *   N              columns covered by the slices; slice_offsets[S] == N.
 *   h              device [T][ldh], ldh >= S*R, sorted order (the output of lora_shrink).
 *   w_b            device [L*N][ldb], ldb >= R: row a*N + n holds B[a][n][:]. Entries with
 *                  j >= lora_ranks[a] never reach the result: the kernels may load them with
 *                  their row (within the first R entries) and zero them before use, so NaN or
 *                  garbage there is harmless.
 *   slice_offsets  device int32 [S+1]: 0 <= slice_offsets[0] <= ... <= slice_offsets[S] = N.
 *   scalings       device float32 [L] (alpha / rank of each adapter).
 *   y              device [T][ldy] read and written in place, ldy >= N; row t is token t.
 *                  (A pitch a little above N, such as N + 256 for N = 6144, measured 4-5%
 *                  faster than ldy = N from 4096 tokens on MI355X.)
 *   workspace      device scratch of lora_expand_workspace_size(...) bytes (the segment
 *                  schedule for many segments; nonzero only then), 16-byte aligned; not read
 *                  before written.
 */
lora_status lora_expand(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t L, int32_t G,
                        int64_t N, const void* h, int64_t ldh, const void* w_b, int64_t ldb,
                        const int32_t* slice_offsets, const int32_t* seg_indptr,
                        const int32_t* weight_indices, const int32_t* permutation,
                        const int32_t* lora_ranks, const float* scalings, void* y, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream);

size_t lora_expand_workspace_size(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t G,
                                  int64_t N);

/* lora_expand with an explicit plan (NULL: as lora_expand); lora_expand_workspace_size covers
 * every plan. */
lora_status lora_expand_ex(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t L,
                           int32_t G, int64_t N, const void* h, int64_t ldh, const void* w_b,
                           int64_t ldb, const int32_t* slice_offsets, const int32_t* seg_indptr,
                           const int32_t* weight_indices, const int32_t* permutation,
                           const int32_t* lora_ranks, const float* scalings, void* y,
                           int64_t ldy, const lora_plan* plan, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * lora_shrink_expand -- lora_shrink followed by lora_expand on the same segments, in one call
 * ("Decode LoRA kernels are optimized", Summary: the chunked shrink -> expand pipeline of one
 * LoRA layer, scheduled on the device with no host synchronisation).
 *
 * Writes h exactly as lora_shrink does and updates y exactly as lora_expand does with that h:
 * every argument has the meaning, layout and range it has there (K, x, w_a, lda as for
 * lora_shrink; N, w_b, ldb, slice_offsets, scalings, y, ldy as for lora_expand; h is the output
 * of the first step and the input of the second). Results are bit-identical to the two calls.
 *
 * At decode sizes both steps run in ONE launch: 16-bit types, T < 1024, ceil(T/16) + G <= 192,
 * K % 8 == 0, R <= 32, a slice layout whose 16-column blocks number a multiple of 3, 16-byte
 * aligned x, w_a, h and w_b rows, R * element size a multiple of 16 bytes, lora_shrink splitting
 * the K reduction of each tile over several workgroups at these sizes, and a grid that is
 * resident on the GPU all at once. The shrink workgroups come first in the launch and count their
 * pieces in on per-tile counters in the workspace; the expand workgroups prime their y and B
 * loads, wait until their tile's pieces are all in, add the pieces themselves (in the order and
 * with the rounding that give h) and finish. Elsewhere the call makes the two launches of
 * lora_shrink and lora_expand.
 *
 *   workspace  device scratch of lora_shrink_expand_workspace_size(...) bytes (never 0 for
 *              T, G > 0), 16-byte aligned. Its first 32 KiB hold counters and MUST be zero
 *              before the first call that uses the workspace; every call leaves them zero
 *              again, so one workspace (sized for the largest call) is reused across calls of
 *              any size, lora_shrink calls and graph replays with no clearing. Calls that
 *              overlap in time must not share it.
 *              The int at byte offset LORA_SHRINK_EXPAND_FLAG_OFFSET is set to 1 if a wait for
 *              the shrink's pieces ever exceeded its one-second bound (the shrink workgroups
 *              never wait, the single launch is taken only when the whole grid fits on the GPU
 *              at once, and workgroups are dispatched in order, so this does not happen; the
 *              bound only guarantees that every wave ends); the y of that call is then undefined, its
 *              counters may be left nonzero, and the workspace must be zero-filled again before
 *              its next use. The library never clears the flag.
 *
 * Errors: as lora_shrink and lora_expand; LORA_EWORKSPACE for a missing, short or misaligned
 * workspace.
 */
#define LORA_SHRINK_EXPAND_FLAG_OFFSET 32764

lora_status lora_shrink_expand(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                               int32_t L, int32_t G, int64_t N, const void* x, int64_t ldx,
                               const void* w_a, int64_t lda, const void* w_b, int64_t ldb,
                               const int32_t* slice_offsets, const int32_t* seg_indptr,
                               const int32_t* weight_indices, const int32_t* permutation,
                               const int32_t* lora_ranks, const float* scalings, void* h,
                               int64_t ldh, void* y, int64_t ldy, void* workspace,
                               size_t workspace_bytes, void* stream);

size_t lora_shrink_expand_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S,
                                         int32_t R, int32_t G, int64_t N);

/*
 * lora_mlp_fused -- single-adapter LoRA MLP with fused SwiGLU (bf16).
 *
 *   out = round( hmid W_d^T + scale * xa_d B_d^T ),      xa_d = round( hmid A_d^T ),
 *   hmid = round( silu(g) * u ),  silu(z) = z / (1 + exp(-z)),
 *   g = x W_g^T + scale * xa_g B_g^T,   u = x W_u^T + scale * xa_u B_u^T,
 *   xa_g = round( x A_g^T ),  xa_u = round( x A_u^T ),
 * with fp32 accumulation and round-to-nearest-even to bf16 at exactly the stored tensors named
 * (xa_*, hmid, out). The scale multiplies the LoRA-B weights in bf16; this is exact for a
 * power-of-two scale (alpha / rank usually is), otherwise s*B_* carries one extra rounding.
 * Dropout 0, no bias, unmerged weights: the conditions of the fast path this implements.
 *
 *   dtype        LORA_BF16 only (others: LORA_EUNSUPPORTED).
 *   M, H, I      tokens, hidden size, intermediate size; H and I multiples of 32; M == 0 no-op.
 *   r            LoRA rank, 1 <= r <= 64.
 *   x            device [M][ldx], ldx >= H, 16-byte aligned rows.
 *   w_gate, w_up device [I][H] contiguous (nn.Linear layout), 16-byte aligned.
 *   w_down       device [H][I] contiguous, 16-byte aligned.
 *   a_gate, a_up device [r][H]; b_gate, b_up device [I][r]; a_down device [r][I];
 *   b_down       device [H][r]; all contiguous, any alignment.
 *   out          device [M][ldo], ldo >= H; written, not read.
 *   workspace    device, >= lora_mlp_workspace_size(...) bytes, 16-byte aligned (holds hmid:
 *                M*I bf16, plus small LoRA buffers). Contents undefined afterwards.
 */
lora_status lora_mlp_fused(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                           float scale, const void* x, int64_t ldx, const void* w_gate,
                           const void* w_up, const void* w_down, const void* a_gate,
                           const void* b_gate, const void* a_up, const void* b_up,
                           const void* a_down, const void* b_down, void* out, int64_t ldo,
                           void* workspace, size_t workspace_bytes, void* stream);

size_t lora_mlp_workspace_size(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r);

/*
 * lora_mlp_fused_train -- lora_mlp_fused that also stores what the backward needs: the gate and
 * up pre-activations e = round(g), v = round(u) (bf16 [M][lde], lde >= I), the saved gate and up
 * projections of the fast path's backward ("Add optional fast lora path for qwen2/qwen3 on npu",
 * review thread: the backward reads the saved X and gate/up projections). out is computed exactly
 * as by lora_mlp_fused; the same workspace size applies. Errors as lora_mlp_fused, plus
 * LORA_EINVAL for a NULL e or v or lde < I.
 */
lora_status lora_mlp_fused_train(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                                 float scale, const void* x, int64_t ldx, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* a_gate,
                                 const void* b_gate, const void* a_up, const void* b_up,
                                 const void* a_down, const void* b_down, void* out, int64_t ldo,
                                 void* e, void* v, int64_t lde, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * lora_mlp_prepare_backward -- the frozen weights in the layout the backward reads, written once
 * per layer (the weights take no gradient): w_gu_t = [W_g^T | W_u^T] as bf16 [H][2I] and
 * w_down_t = W_d^T as bf16 [I][H], both packed and 16-byte aligned, from the nn.Linear weights
 * w_gate, w_up [I][H] and w_down [H][I] (packed). The backward's products then reduce over
 * contiguous rows as the forward's do. Errors: LORA_EUNSUPPORTED for a dtype other than bf16,
 * LORA_EINVAL for a NULL pointer or H, I < 1.
 */
lora_status lora_mlp_prepare_backward(lora_dtype dtype, int64_t H, int64_t I, const void* w_gate,
                                      const void* w_up, const void* w_down, void* w_gu_t,
                                      void* w_down_t, void* stream);

/*
 * lora_mlp_backward -- gradients of the single-adapter LoRA MLP with SwiGLU (bf16) for the fast
 * path's backward ("Add optional fast lora path for qwen2/qwen3 on npu", review thread and
 * Verification advice: SwiGLU backward from the saved gate/up projections, dX from df and the
 * weights, LoRA A/B gradients, X never overwritten; the page shows fragments only, this is its
 * reading). With d = dout, f = silu(e):
 *
 *   hmid = round(f v), xa_g = round(x A_g^T), xa_u = round(x A_u^T), xa_d = round(hmid A_d^T),
 *   dxa_d = round(s d B_d),   dhmid = d W_d + dxa_d A_d   (fp32, not stored),
 *   de = round(dhmid v silu'(e)),  dv = round(dhmid f),
 *   dxa_g = round(s de B_g),  dxa_u = round(s dv B_u),
 *   dx = round(de W_g + dv W_u + dxa_g A_g + dxa_u A_u),
 *   da_down = round(dxa_d^T hmid), db_down = round(s d^T xa_d),
 *   da_gate = round(dxa_g^T x),    db_gate = round(s de^T xa_g),  (up likewise)
 *
 * silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))); fp32 accumulation; s is folded into bf16
 * copies of B (exact for a power of two). The frozen W take no gradient.
 *
 *   x [M][ldx], dout [M][lddo]: 16-byte aligned rows. e, v [M][lde] from lora_mlp_fused_train
 *   (16-byte aligned rows).
 *   w_gu_t, w_down_t: from lora_mlp_prepare_backward. a_*, b_* as for lora_mlp_fused.
 *   dx [M][lddx] (must not be x or dout); da_gate, da_up [r][H]; db_gate, db_up [I][r];
 *   da_down [r][I]; db_down [H][r]: all bf16, packed, written (not accumulated).
 *   workspace    device, >= lora_mlp_backward_workspace_size(...) bytes, 16-byte aligned.
 * Requires H and I multiples of 32 and 1 <= r <= 64 (else LORA_EUNSUPPORTED). Nothing is read on
 * the host; every launch is on `stream`.
 */
lora_status lora_mlp_backward(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                              float scale, const void* x, int64_t ldx, const void* e,
                              const void* v, int64_t lde, const void* dout, int64_t lddo,
                              const void* w_gu_t, const void* w_down_t, const void* a_gate,
                              const void* b_gate, const void* a_up, const void* b_up,
                              const void* a_down, const void* b_down, void* dx, int64_t lddx,
                              void* da_gate, void* db_gate, void* da_up, void* db_up,
                              void* da_down, void* db_down, void* workspace,
                              size_t workspace_bytes, void* stream);

size_t lora_mlp_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t H, int64_t I,
                                        int32_t r);

/*
 * lora_mlp_backward_intermediates -- where lora_mlp_backward leaves its stored intermediates in
 * its workspace (valid until the workspace is reused), for inspection and step-by-step checks:
 * byte offsets (16-byte aligned) of bf16 row-major arrays, written to offsets[0..5]:
 *   [0] hmid [M][I]   [1] [de | dv] [M][2I]   [2] [xa_g | xa_u] [M][2 rp]   [3] xa_d [M][rp]
 *   [4] dxa_d [M][rp] [5] [dxa_g | dxa_u] [M][2 rp]
 * where rp, the rank rounded up to 32, is the return value (columns r..rp-1 of each rp block
 * hold zeros). Returns 0 (and writes nothing) for sizes lora_mlp_backward rejects or a NULL
 * offsets pointer.
 */
int32_t lora_mlp_backward_intermediates(int64_t M, int64_t H, int64_t I, int32_t r,
                                        size_t* offsets);

/*
 * lora_linear_fused -- single-adapter LoRA linear projection (bf16): the attention output
 * projection of the fast LoRA path of "Add optional fast lora path for qwen2/qwen3 on npu" (What
 * this PR does: the attention forward with fast LoRA projections; Compatibility checks as for
 * the MLP).
 *
 *   out = round( x W^T + scale * xa B^T ),   xa = round( x A^T ),
 * with fp32 accumulation and round-to-nearest-even to bf16 at xa and out only. The scale is
 * folded into a bf16 copy of B (exact for a power-of-two scale, as for the MLP).
 *
 *   M, K, N        rows of x, input features (K % 32 == 0), output features.
 *   r              LoRA rank, 1 <= r <= 64.
 *   x              device [M][ldx] bf16, ldx >= K, 16-byte aligned rows.
 *   w              device [N][K] bf16, contiguous, 16-byte aligned.
 *   a, b           device [r][K] and [N][r] bf16, contiguous.
 *   out            device [M][ldo] bf16, ldo >= N (a new tensor; not accumulated into).
 *   workspace      device scratch of lora_linear_workspace_size(...) bytes, 16-byte aligned.
 * Returns LORA_EUNSUPPORTED for another dtype, K % 32 != 0, r > 64 or unaligned x / w.
 */
lora_status lora_linear_fused(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r,
                              float scale, const void* x, int64_t ldx, const void* w,
                              const void* a, const void* b, void* out, int64_t ldo,
                              void* workspace, size_t workspace_bytes, void* stream);

size_t lora_linear_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r);

/*
 * lora_qkv_fused -- the query, key and value projections of one x, each a single-adapter LoRA
 * linear projection as in lora_linear_fused (same page and section). The three LoRA-A products
 * are formed in one pass over x; each projection then runs one matrix product with its LoRA
 * term folded into the reduction.
 *
 *   q = round( x W_q^T + scale * round(x A_q^T) B_q^T ),  k and v likewise,
 *   x [M][ldx]; W_q [Nq][K], W_k and W_v [Nkv][K]; A_* [r][K]; B_q [Nq][r], B_k, B_v [Nkv][r];
 *   q [M][ldq >= Nq], k [M][ldk >= Nkv], v [M][ldv >= Nkv]. Other requirements as for
 *   lora_linear_fused; workspace of lora_qkv_workspace_size(...) bytes.
 */
lora_status lora_qkv_fused(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                           int32_t r, float scale, const void* x, int64_t ldx, const void* w_q,
                           const void* w_k, const void* w_v, const void* a_q, const void* b_q,
                           const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                           void* q, int64_t ldq, void* k, int64_t ldk, void* v, int64_t ldv,
                           void* workspace, size_t workspace_bytes, void* stream);

size_t lora_qkv_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                               int32_t r);

/*
 * lora_linear_prepare_backward -- the frozen weight of a projection in the layout
 * lora_linear_backward reads, written once per layer (bf16): w [N][K] (nn.Linear [out][in]) ->
 * w_t [K][N] (W^T, row-major, pitch N). Both device buffers are the caller's.
 */
lora_status lora_linear_prepare_backward(lora_dtype dtype, int64_t K, int64_t N, const void* w,
                                         void* w_t, void* stream);

/*
 * lora_linear_backward -- gradients of the single-adapter LoRA projection (bf16) for the fast
 * path's backward ("Add optional fast lora path for qwen2/qwen3 on npu", Verification advice:
 * gradients of the projection fast paths checked against a reference; What this PR does: the
 * LoRA projections of the attention). For y = x W^T + scale * round(x A^T) B^T and
 * dout = dL/dy, with the forward's rounding points (every stored intermediate and result
 * rounded once to bf16, fp32 accumulation):
 *     xa  = round(x A^T)                     (recomputed)
 *     dxa = round(dout (scale B))
 *     dx  = round(dout W + dxa A)            [M][K]
 *     dA  = round(dxa^T x)                   [r][K]
 *     dB  = round(scale dout^T xa)           [N][r]
 * The frozen W takes no gradient. scale is folded into a bf16 copy of B (exact for a power of
 * two, as alpha / rank usually is).
 *
 *   x [M][ldx >= K] (the saved input, only read); dout [M][lddo >= N]; w_t = W^T [K][N] from
 *   lora_linear_prepare_backward; a [r][K]; b [N][r]; dx [M][lddx >= K], which must not be x or
 *   dout; da [r][K]; db [N][r] (contiguous). 1 <= r <= 64; K and N multiples of 32; x, dout,
 *   w_t 16-byte aligned with 16-byte aligned row pitches. workspace of
 *   lora_linear_backward_workspace_size(...) bytes, 16-byte aligned, not read before written.
 * Errors: LORA_EINVAL (sizes, null pointers, pitches, dx aliasing an input),
 * LORA_EUNSUPPORTED (dtype, rank, multiples, alignment), LORA_EWORKSPACE, LORA_EHIP.
 */
lora_status lora_linear_backward(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r,
                                 float scale, const void* x, int64_t ldx, const void* dout,
                                 int64_t lddo, const void* w_t, const void* a, const void* b,
                                 void* dx, int64_t lddx, void* da, void* db, void* workspace,
                                 size_t workspace_bytes, void* stream);

size_t lora_linear_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t N,
                                           int32_t r);

/*
 * lora_qkv_prepare_backward -- the frozen query, key and value weights in the layout
 * lora_qkv_backward reads, written once per layer (bf16): w_q [Nq][K], w_k and w_v [Nkv][K] ->
 * w_qkv_t = [W_q^T | W_k^T | W_v^T] [K][Nq + 2 Nkv] (row-major). Buffers are the caller's.
 */
lora_status lora_qkv_prepare_backward(lora_dtype dtype, int64_t K, int64_t Nq, int64_t Nkv,
                                      const void* w_q, const void* w_k, const void* w_v,
                                      void* w_qkv_t, void* stream);

/*
 * lora_qkv_backward -- gradients of lora_qkv_fused (bf16): the query, key and value projections
 * of one x, each as lora_linear_backward, with the three projections' contributions to dx summed
 * in fp32 and rounded once (same source as lora_linear_backward):
 *     dx = round( sum_{p in q,k,v} dout_p W_p + dxa_p A_p ),   dxa_p = round(dout_p (scale B_p))
 *     dA_p = round(dxa_p^T x),   dB_p = round(scale dout_p^T xa_p),   xa_p = round(x A_p^T)
 *
 *   x [M][ldx >= K]; dq [M][lddq >= Nq], dk [M][lddk >= Nkv], dv [M][lddv >= Nkv]; w_qkv_t from
 *   lora_qkv_prepare_backward; a_* [r][K]; b_q [Nq][r], b_k and b_v [Nkv][r]; dx [M][lddx >= K]
 *   (not x, dq, dk or dv); da_* [r][K]; db_q [Nq][r], db_k and db_v [Nkv][r] (contiguous).
 *   1 <= r <= 64; K, Nq and Nkv multiples of 32; x, dq, dk, dv and w_qkv_t 16-byte aligned with
 *   16-byte aligned row pitches. workspace of lora_qkv_backward_workspace_size(...) bytes,
 *   16-byte aligned, not read before written (it also holds [dq | dk | dv] side by side for the
 *   dx product; when dk == dq + Nq and dv == dk + Nkv elements with one row pitch -- column views
 *   of the gradient of a fused q/k/v output -- they are read in place instead).
 * Errors as lora_linear_backward.
 */
lora_status lora_qkv_backward(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                              int32_t r, float scale, const void* x, int64_t ldx, const void* dq,
                              int64_t lddq, const void* dk, int64_t lddk, const void* dv,
                              int64_t lddv, const void* w_qkv_t, const void* a_q, const void* b_q,
                              const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                              void* dx, int64_t lddx, void* da_q, void* db_q, void* da_k,
                              void* db_k, void* da_v, void* db_v, void* workspace,
                              size_t workspace_bytes, void* stream);

size_t lora_qkv_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq,
                                        int64_t Nkv, int32_t r);

/*
 * lora_embedding_a -- the LoRA-A product of an embedding layer (the embedding LoRA-A forward of
 * "Decode LoRA kernels are optimized", Summary and Behaviour changes; the page does not print
 * the arithmetic, this is its reading): for segment g (adapter a, rank r = lora_ranks[a]) and
 * sorted position i in it,
 *     h[i][j] = A[a][j][input_ids[permutation[i]]]   for j < r,   0 for r <= j < R,
 * the column of the adapter's A at the token's vocabulary id (one-hot row times A^T), copied
 * bit for bit. No longest-segment bound is needed: the launch is sized from T and G on the host
 * and no call reads device memory on the host. Rows of h that no segment covers are not written.
 *
 *   dtype          element type of A and h.
 *   T, V, R, L, G  tokens, vocabulary size, padded rank (1 <= R <= 1024), adapters, segments.
 *   input_ids      device int32 [T] in token order. An id outside [0, V) is a caller error: its
 *                  row of h gets zeros and A is not read for it.
 *   w_a            device; A[a][j][v] is the element at a*stride_l + j*stride_r + v*stride_v
 *                  (element strides; stride_l >= 0, stride_r >= 1, stride_v >= 1). [L][R][V]
 *                  storage has stride_v = 1; [L][V][R] storage (stride_r = 1) makes each token's
 *                  values one contiguous run, the faster layout. Elements with j >= lora_ranks[a]
 *                  are never read. The strides must keep every read inside the caller's buffer.
 *   seg_indptr, weight_indices, permutation (NULL: identity), lora_ranks: as for lora_shrink
 *                  (an adapter index or permutation entry out of range also gives a zero row).
 *   h              device [T][ldh], ldh >= R, sorted order.
 * One kernel launch of ceil(T / 256) workgroups; no workspace for any segment count.
 */
lora_status lora_embedding_a(lora_dtype dtype, int64_t T, int64_t V, int32_t R, int32_t L,
                             int32_t G, const int32_t* input_ids, const void* w_a,
                             int64_t stride_l, int64_t stride_r, int64_t stride_v,
                             const int32_t* seg_indptr, const int32_t* weight_indices,
                             const int32_t* permutation, const int32_t* lora_ranks, void* h,
                             int64_t ldh, void* stream);

/*
 * lora_check_metadata -- the value checks of the LoRA metadata that "Decode LoRA kernels are
 * optimized" (Behaviour changes) takes off the fast path, as an explicit call that waits for its
 * own result (it synchronizes `stream`; not for capture). Rules, reported as the first one broken:
 *   1 seg_indptr [G+1]: starts at 0, never decreases, ends at T;
 *   2 weight_indices [G]: inside [0, L);
 *   3 lora_ranks [L]: inside [0, R];
 *   4 permutation [T] (NULL: not checked, the identity): every value in [0, T) exactly once;
 *   5 slice_offsets [S+1] (NULL: not checked): start >= 0, never decrease, end at N.
 * Returns LORA_OK, or LORA_EVALUE with *rule (host int, may be NULL) set to the rule number (0
 * when valid). Every device access is bounded by the sizes, so any values are safe to check.
 * workspace: device, >= lora_check_metadata_workspace_size(T) bytes, 16-byte aligned.
 * Errors: LORA_EINVAL (negative size, NULL seg_indptr, or NULL weight_indices / lora_ranks with
 * G / L > 0), LORA_EWORKSPACE, LORA_EHIP.
 */
lora_status lora_check_metadata(int64_t T, int32_t G, int32_t L, int32_t R, int32_t S, int64_t N,
                                const int32_t* seg_indptr, const int32_t* weight_indices,
                                const int32_t* permutation, const int32_t* lora_ranks,
                                const int32_t* slice_offsets, int32_t* rule, void* workspace,
                                size_t workspace_bytes, void* stream);

size_t lora_check_metadata_workspace_size(int64_t T);

/*
 * lora_schedule_tiles -- the segment schedule the compute kernels use, exported for checking.
 *
 * Each non-empty segment g is cut into row tiles of at most BM sorted positions starting at
 * seg_indptr[g]; empty segments give none. The list is segment-major with ascending starts.
 * Writes tiles[5*t + {0..4}] = {g, m0, mlen, a, r} (a = weight_indices[g], r = lora_ranks[a])
 * for t < *count, and *count.
 *
 *   BM         tile height, 1 <= BM <= 4096.
 *   method     0: the per-workgroup search the kernels run inline; 1: the standalone scheduler
 *              kernel used when G is large. Both must give the same list.
 *   tiles      device int32 [max_tiles][5]; max_tiles >= T/BM + G (rounded up) suffices.
 *   count      device int32 [1].
 *   workspace  device scratch of at least 16*(ceil(T/BM) + G) + 256 bytes for method 1.
 */
lora_status lora_schedule_tiles(int64_t T, int32_t G, int32_t BM, int32_t method,
                                const int32_t* seg_indptr, const int32_t* weight_indices,
                                const int32_t* lora_ranks, int32_t* tiles, int64_t max_tiles,
                                int32_t* count, void* workspace, size_t workspace_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
