/*
 * ikbo.h -- C ABI of libikbo: the IKBO Linear Compression Embedding forward (and its
 * backward) on AMD Instinct MI355X (gfx950).
 *
 * The operation (IKBO recsys blog, "Deep Dive: Linear Compression"; aibriefing
 * article, "kernel deep-dive case 1"):
 *
 *     Y[b] = W_u . U[map[b]]  +  W_c . C[b]          for b < B_c
 *
 * U holds the request-only (user) embeddings at their own batch B_u, C the
 * per-candidate embeddings at batch B_c, and map[b] names the user of
 * candidate b.  The kernels take the two batches "in their natural, mismatched
 * sizes" plus the candidate-to-user map (blog, "Why broadcast is a data-layout
 * problem" and "How the IKBO co-design is built"; aibriefing, RO/NRO paragraph)
 * and never build the replicated tensor U[map].
 *
 * Layouts.  Every tensor is dense row-major (C order) in device memory owned by
 * the caller:
 *     U   [B_u, K_u, D]      C   [B_c, K_c, D]      map [B_c] int32
 *     W_u [M, K_u]           W_c [M, K_c]           Y   [B_c, M, D]
 * U, C, W_u, W_c and Y share one element type (bfloat16 or float32).  Products
 * accumulate in float32; the user partial W_u.U[u] is kept in float32; Y is
 * rounded once (round-to-nearest-even) when it is stored.
 *
 * Threading.  A plan may be used from one host thread and one stream at a
 * time.  Different plans are independent.  No C++ exception crosses this ABI.
 */
#ifndef IKBO_H
#define IKBO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque plan handle; created by ikbo_lce_plan, owned by the library. */
typedef struct ikbo_lce_plan_s *ikbo_lce_plan_t;

/* Status codes returned by every entry point. */
enum {
    IKBO_OK = 0,
    IKBO_ERR_INVALID_ARG = -1,  /* null pointer, bad dimension, shape differs from the plan */
    IKBO_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. D*elt not a multiple of 16 B) */
    IKBO_ERR_HIP = -3,          /* a HIP runtime call failed; see ikbo_last_error_message() */
    IKBO_ERR_ALIGNMENT = -4,    /* a tensor base address is not 16-byte aligned */
    IKBO_ERR_TIMEOUT = -5,      /* device: a candidate tile gave up waiting for its user partial */
    IKBO_ERR_MAP_RANGE = -6     /* device: some map[b] lies outside [0, B_u) */
};

/* Element type of U, C, W_u, W_c and Y. */
enum { IKBO_DTYPE_BF16 = 0, IKBO_DTYPE_F32 = 1 };

/*
 * Kernel variant.  S0..S4 reproduce the pages' optimisation ladder on CDNA4
 * (blog, "Deep Dive: Linear Compression", stages 1-4; zubnet summary, the
 * four-stage paragraph); all five compute the same Y.
 *   S0  materialise X = [U[map] ; C] in HBM, then one batched GEMM with [W_u | W_c];
 *   S1  decompose by linearity (user GEMM at B_u rows, candidate GEMM at B_c rows),
 *       then materialise P_u[map] and add; unpadded K, 4-byte operand loads;
 *   S2  S1 with K zero-padded and 16-byte operand loads;
 *   S3  user GEMM, then a candidate GEMM whose epilogue gathers P_u[map[b]] by
 *       index and adds it in registers;
 *   S4  one launch: user and candidate tiles overlap, candidate epilogues wait for
 *       their user partial through device-scope release/acquire flags.
 * AUTO selects S4.
 */
enum {
    IKBO_VARIANT_AUTO = 0,
    IKBO_S0_MATERIALISED = 1,
    IKBO_S1_DECOMPOSED = 2,
    IKBO_S2_ALIGNED = 3,
    IKBO_S3_EPILOGUE_FUSED = 4,
    IKBO_S4_PERSISTENT = 5
};

/* Plan flags (host-forced test conditions; production callers pass 0). */
enum {
    IKBO_FLAG_DEBUG_DELAY_USER = 2, /* S4: user tiles sleep before computing (exercises the wait) */
    IKBO_FLAG_DEBUG_SKIP_USER = 4,  /* S4: user tiles publish nothing; candidates time out */
    IKBO_FLAG_BACKWARD = 8,         /* also allocate the workspace of ikbo_lce_backward */
    IKBO_FLAG_DEBUG_POISON_USER = 16 /* each forward first fills the user partials P_u with NaN */
};

/*
 * Create a plan for one shape range ("the compiler needs each operator's
 * dynamic shape range to pick the kernel": blog, co-design section; aibriefing,
 * three-layers paragraph).  Chooses the tile configuration and allocates the
 * device workspace (hipMalloc) on the current device; forward never allocates.
 *   max_B_u, max_B_c  upper bounds of B_u and B_c in later forwards (>= 1, >= 0)
 *   K_u, K_c, M, D    fixed dimensions (>= 1)
 *   dtype             IKBO_DTYPE_*
 *   variant           IKBO_VARIANT_AUTO or IKBO_S*
 * On success stores a handle in *plan and returns IKBO_OK; on failure *plan is
 * left NULL and nothing stays allocated.  Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
int ikbo_lce_plan(ikbo_lce_plan_t *plan, int max_B_u, int max_B_c, int K_u, int K_c,
                  int M, int D, int dtype, int variant, unsigned flags);

/*
 * Enqueue Y[b] = W_u.U[map[b]] + W_c.C[b] on `stream` (a hipStream_t; NULL =
 * the null stream).  All pointers are device pointers with the layouts above;
 * U, C, W_u, W_c and Y must be 16-byte aligned.  The dimensions must equal the
 * plan's, with 1 <= B_u <= max_B_u and 0 <= B_c <= max_B_c; B_c = 0 is a no-op.
 * Host-side validation errors return before anything is enqueued.  The call is
 * asynchronous: device-side conditions (map entry out of range, S4 wait
 * timeout) are recorded in the plan and reported by ikbo_lce_check; the Y rows
 * of an affected candidate are then unspecified.  Must be called with the
 * plan's device current.
 */
int ikbo_lce_forward(ikbo_lce_plan_t plan, const void *U, const void *C, const int32_t *map,
                     const void *W_u, const void *W_c, void *Y,
                     int B_u, int B_c, int K_u, int K_c, int M, int D, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the forward above without
 * a plan, calling no hipMalloc, hipFree or other allocating routine.  It computes
 * the same Y as the two-launch gather-add stage (S3) on the streaming engine, and
 * keeps the float32 user partial P_u [B_u, M, D] in a file-scope device array of
 * IKBO_NOALLOC_SCRATCH_BYTES bytes (256 of them reserved) that every GPU the
 * library runs on holds until the process ends.  Limits: bf16 only, D in
 * {32, 64, 128, 160, 192}, and B_u*M*D*4 <= IKBO_NOALLOC_SCRATCH_BYTES - 256;
 * beyond them it returns IKBO_ERR_UNSUPPORTED (ikbo_last_error_message says which)
 * before anything is enqueued.  Arguments, layouts, alignment and the other errors
 * are those of ikbo_lce_forward (the dimensions are not checked against a plan).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two host threads) race and may produce wrong Y.  Map entries
 * outside [0, B_u) leave their candidates' Y rows unwritten; this entry point does
 * not report them.  The first call on a device also looks up the array's device
 * address (no allocation).
 */
#define IKBO_NOALLOC_SCRATCH_BYTES (8u << 20)
int ikbo_lce_forward_noalloc(const void *U, const void *C, const int32_t *map,
                             const void *W_u, const void *W_c, void *Y,
                             int B_u, int B_c, int K_u, int K_c, int M, int D, void *stream);

/*
 * Enqueue the gradients of L = <dY, Y> for the forward above (the chain rule of the
 * pages' definition, blog "Deep Dive: Linear Compression", stage 1; the aibriefing
 * article's three-layers paragraph says the kernels serve training when the ratio
 * exceeds 1, but the pages give no training formulas):
 *
 *     dC[b] = W_c^T . dY[b]                    dW_c = sum_b dY[b] . C[b]^T
 *     dU[u] = W_u^T . S[u]                     dW_u = sum_b dY[b] . U[map[b]]^T
 *     S[u]  = sum of dY[b] over the candidates b with map[b] = u
 *
 * The replicated user tensor is not built in this direction either: the user
 * gradient is summed per user first and multiplied at batch B_u.  Requires a plan
 * made with IKBO_FLAG_BACKWARD (bf16, D in {32, 64, 128, 160, 192}; otherwise the
 * plan call returns IKBO_ERR_UNSUPPORTED); the variant does not matter.
 * Layouts (device memory owned by the caller, dense row-major):
 *     dY [B_c, M, D] bf16 (input)         U, C, map, W_u, W_c as for the forward
 *     dU [B_u, K_u, D] bf16 (output)      dC [B_c, K_c, D] bf16 (output)
 *     dW_u [M, K_u] float32 (output)      dW_c [M, K_c] float32 (output)
 * Every output is overwritten, not accumulated into; users that no candidate maps to
 * get dU = 0, and B_c = 0 gives dU = 0 and dW = 0 (dY, C, map and dC may then be NULL).
 * Products accumulate in float32; S is kept in float32 and handed to the bf16 matrix
 * cores as the pair bf16(S) + bf16(S - bf16(S)); dU and dC are rounded once to bf16.
 * Every pointer except map must be 16-byte aligned (map: 4-byte).  Asynchronous, like
 * the forward: map entries outside [0, B_u) are skipped and reported by ikbo_lce_check
 * as IKBO_ERR_MAP_RANGE.  Uses the plan's workspace: do not overlap it with a forward
 * or another backward on the same plan in a different stream.  dC and dU run on two
 * streams that the plan owns, forked from `stream` by events after the work they need
 * and joined back into it before the call returns: work enqueued on `stream` afterwards
 * sees every output (under stream capture the fork and join are captured with it).
 * Errors (before anything is enqueued): INVALID_ARG, ALIGNMENT, UNSUPPORTED, HIP.
 */
int ikbo_lce_backward(ikbo_lce_plan_t plan, const void *dY, const void *U, const void *C,
                      const int32_t *map, const void *W_u, const void *W_c, void *dU, void *dC,
                      float *dW_u, float *dW_c, int B_u, int B_c, int K_u, int K_c, int M, int D,
                      void *stream);

/*
 * Wait for `stream`, then return and clear the device-side status recorded by
 * earlier forwards and backwards on this plan (IKBO_OK, IKBO_ERR_MAP_RANGE or
 * IKBO_ERR_TIMEOUT), or IKBO_ERR_HIP if the wait itself failed.
 */
int ikbo_lce_check(ikbo_lce_plan_t plan, void *stream);

/*
 * Write a NUL-terminated JSON description of the plan (variant, tile sizes,
 * padded K, grid, workspace bytes) into json[0..cap).  Returns the length it
 * needed (excluding the NUL), or a negative status.
 */
int ikbo_lce_plan_info(ikbo_lce_plan_t plan, char *json, size_t cap);

/*
 * Upper bound on the polling iterations a candidate tile spends waiting for a
 * user partial (S4) before it records IKBO_ERR_TIMEOUT and moves on; 0 restores
 * the default.  A test hook: every kernel exits even if a user tile never
 * publishes.
 */
int ikbo_lce_plan_set_spin_limit(ikbo_lce_plan_t plan, uint32_t max_polls);

/* Free the plan and its workspace (synchronises the device first).  NULL is a no-op. */
int ikbo_lce_plan_destroy(ikbo_lce_plan_t plan);

/*
 * IKBO target attention (IKBO recsys blog, "Deep Dive: Flash Attention"): the queries of
 * each candidate attend over the keys and values of its user,
 *
 *     O[b,h] = softmax(scale * Q[b,h] . K[map[b],h]^T) . V[map[b],h]      for b < B_c, h < H
 *
 * with K and V at the user batch B_u, never replicated per candidate.  Layouts (device
 * memory owned by the caller, dense row-major, bf16):
 *     Q, O [B_c, H, L_q, head_dim]      K, V [B_u, H, L_kv, head_dim]      map [B_c] int32
 * Scores, softmax and the weighted sum accumulate in float32 (the softmax weights reach
 * the matrix cores as bf16); O is rounded to bf16 once.  No mask: every query sees all
 * L_kv keys of its user.
 *
 * ikbo_fa_plan: fixed H, L_q, L_kv, head_dim; bf16 only, head_dim 64 or 128, L_q 16, 32
 * or 64 (one wave holds a candidate's queries); any L_kv >= 1.  flags must be 0.
 * Allocates a small workspace (the candidates grouped by user) on the current device.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
typedef struct ikbo_fa_plan_s *ikbo_fa_plan_t;
int ikbo_fa_plan(ikbo_fa_plan_t *plan, int max_B_u, int max_B_c, int H, int L_q, int L_kv, int head_dim,
                 int dtype, unsigned flags);

/*
 * Enqueue the attention on `stream`.  scale = 0 means 1/sqrt(head_dim); a negative, NaN or
 * infinite scale is INVALID_ARG.  Q, K, V and O must be 16-byte aligned, map 4-byte.
 * B_c = 0 is a no-op.  Asynchronous: map entries outside [0, B_u) leave their candidates'
 * O unwritten and are reported by ikbo_fa_check as IKBO_ERR_MAP_RANGE.  One plan serves
 * one stream at a time.
 */
int ikbo_fa_forward(ikbo_fa_plan_t plan, const void *Q, const void *K, const void *V, const int32_t *map,
                    void *O, int B_u, int B_c, int H, int L_q, int L_kv, int head_dim, float scale,
                    void *stream);

/*
 * Self + target attention in one launch (blog, "Self + Target Attention Fusion"): besides the
 * candidates' target attention above, the user sequence's own queries attend over the same K
 * and V (no mask, like the target queries):
 *
 *     O_self[u,h] = softmax(scale * Q_self[u,h] . K[u,h]^T) . V[u,h]        for u < B_u
 *
 * Q_self, O_self [B_u, H, L_self, head_dim] bf16 (16-byte aligned); L_self a multiple of L_q
 * (the self queries are taken L_q at a time, as further work of their user, so they share the
 * K/V blocks the user's candidates stage).  L_self = 0 is ikbo_fa_forward; B_c = 0 computes
 * only the self part (Q, map and O may then be NULL).  Otherwise as ikbo_fa_forward.
 */
int ikbo_fa_forward_fused(ikbo_fa_plan_t plan, const void *Q, const void *K, const void *V,
                          const int32_t *map, void *O, const void *Q_self, void *O_self, int B_u,
                          int B_c, int H, int L_q, int L_kv, int L_self, int head_dim, float scale,
                          void *stream);

/* Wait for `stream`, then return and clear the device status (IKBO_OK or IKBO_ERR_MAP_RANGE). */
int ikbo_fa_check(ikbo_fa_plan_t plan, void *stream);

/* Free the plan and its workspace (synchronises the device first).  NULL is a no-op. */
int ikbo_fa_plan_destroy(ikbo_fa_plan_t plan);

/* Static text for a status code. */
const char *ikbo_status_str(int status);

/* Text of the last IKBO_ERR_HIP failure seen by the calling host thread ("" if none). */
const char *ikbo_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* IKBO_H */
