/*
 * jvpattn: fused attention forward carrying dual numbers, for AMD Instinct
 * MI355X (gfx950).
 *
 * What it computes. Given queries Q, keys K, values V and their tangents
 * dQ, dK, dV (all [B, H, N, d], d fastest), one call returns
 *
 *   O    = softmax(scale * Q K^T + M) V               attention output
 *   dO   = d/dt O(Q + t dQ, K + t dK, V + t dV) at 0   its Jacobian-vector product
 *   lse  = logsumexp_j(scale * Q K^T + M)             natural log, per query row
 *   tlse = sum_j P_ij dS_ij,  dS = scale (dQ K^T + Q dK^T)   (the JVP of lse)
 *
 * The operation is the one the "JVP Flash Attention" README describes: a
 * drop-in for PyTorch's scaled_dot_product_attention (section "Usage":
 * q, k, v and attn_mask, no dropout) that supports Jacobian-vector products
 * (section "Description"). The per-head computation is the plain scaled
 * dot-product attention of the naive MHSA script in the equinox issue
 * "Flash Attention" (#732): scores divided by sqrt(key depth) by default,
 * softmax over keys, weights applied to V.
 *
 * Conventions (the pages leave these open; these are SDPA's):
 *   - boolean mask: nonzero = the key takes part, zero = excluded;
 *   - additive mask: added after scaling, treated as a constant (no tangent);
 *   - causal: key j is visible to query i iff j <= i (top-left aligned); with
 *     a mask as well, both restrictions apply;
 *   - a query row with no visible key gets O = dO = 0, lse = -inf, tlse = 0.
 *
 * All pointers other than `params` are device pointers (HBM) owned by the
 * caller. Nothing is allocated and no state is kept between calls beyond the
 * loaded code objects. Work is queued on `stream` (a hipStream_t; NULL is the
 * null stream) and the call returns without waiting for it.
 */
#ifndef JVPATTN_H
#define JVPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. One type applies to q, k, v, dq, dk, dv, o, do and, for
 * JVPATTN_MASK_ADDITIVE, to the mask. */
typedef enum {
  JVPATTN_F32 = 0,   /* IEEE float32 */
  JVPATTN_F16 = 1,   /* IEEE float16 */
  JVPATTN_BF16 = 2   /* bfloat16 */
} jvpattn_dtype;

typedef enum {
  JVPATTN_MASK_NONE = 0,
  JVPATTN_MASK_BOOL = 1,      /* uint8 (torch.bool): nonzero = attend */
  JVPATTN_MASK_ADDITIVE = 2,  /* the element type above, added to scaled scores */
  JVPATTN_MASK_BITS = 3       /* a boolean mask, one bit per key: uint32 words, key j of a row
                                 attends iff bit (j % 32) of the row's word j / 32 is set;
                                 ceil(Nk / 32) words per row */
} jvpattn_mask_kind;

/* Return codes. Every error is detected before any work is queued, so a
 * call that fails writes nothing -- except JVPATTN_ERR_HIP, which reports a
 * failed kernel launch. No error crosses the interface as an exception. */
enum {
  JVPATTN_OK = 0,
  JVPATTN_ERR_NULL = -1,     /* a required pointer is NULL */
  JVPATTN_ERR_SHAPE = -2,    /* B, H, Nq, Nk < 0, Hkv < 0 or not a divisor of H, a size overflows
                                int64, B*H > INT32_MAX, or one head of q or k (N*d*element size)
                                exceeds 2 GiB */
  JVPATTN_ERR_DTYPE = -3,    /* dtype not one of jvpattn_dtype */
  JVPATTN_ERR_HEADDIM = -4,  /* d not supported (forward: 32, 64, 96, 128, and 256 for float16 /
                                bfloat16; reverse pass: 64) */
  JVPATTN_ERR_MASK = -5,     /* mask_kind unknown, mask NULL/non-NULL mismatch, negative strides,
                                or one head's mask slice exceeds 2 GiB */
  JVPATTN_ERR_ALIGN = -6,    /* a tensor pointer not 16-byte aligned (lse/tlse: 4-byte) */
  JVPATTN_ERR_SCALE = -7,    /* scale not finite or not > 0 */
  JVPATTN_ERR_ALIAS = -8,    /* an output overlaps an input or another output */
  JVPATTN_ERR_HIP = -9,      /* the HIP runtime reported an error on launch */
  JVPATTN_ERR_WORKSPACE = -10, /* jvpattn_bwd: workspace NULL, too small, misaligned, or overlapping */
  JVPATTN_ERR_ARG = -11,       /* jvpattn_fwd_set_algo: a value outside its documented range */
  JVPATTN_ERR_SCRATCH = -12    /* jvpattn_bwd_noalloc: B*H*Nq exceeds JVPATTN_BWD_NOALLOC_MAX_ROWS */
};

typedef struct {
  int32_t B, H;          /* batch, heads */
  int32_t Nq, Nk;        /* query rows, key/value rows (causal is top-left aligned when Nq != Nk) */
  int32_t d;             /* head dimension of q, k, v: 32, 64, 96, 128, or 256 (16-bit types) */
  int32_t dtype;         /* jvpattn_dtype */
  int32_t mask_kind;     /* jvpattn_mask_kind */
  int32_t causal;        /* 0 or 1 */
  /* Mask element (b, h, i, j) is at mask[b*mask_stride_b + h*mask_stride_h
   * + i*mask_stride_q + j] (strides in elements, j contiguous; for
   * JVPATTN_MASK_BITS the elements are the 32-bit words and j the word index).
   * A stride of 0 broadcasts that axis, e.g. a [B,1,Nq,Nk] mask has
   * mask_stride_h = 0 and a key-padding mask [B,1,1,Nk] also has
   * mask_stride_q = 0. Ignored when mask_kind is NONE. */
  int64_t mask_stride_b, mask_stride_h, mask_stride_q;
  float scale;           /* multiplies Q K^T and dQ K^T + Q dK^T; finite and > 0 (SDPA default 1/sqrt(d)) */
  /* Heads of k, v, tk, tv (grouped-query attention, as SDPA's enable_gqa):
   * query head h reads key/value head h / (H / Hkv), so H must be a multiple
   * of Hkv; Hkv = 1 is multi-query attention. 0 is read as H (one key/value
   * head per query head). */
  int32_t Hkv;
} jvpattn_params;

/* Host-only validation of a jvpattn_fwd call: the same checks jvpattn_fwd
 * makes, in the same order, without touching the GPU (pointers are only
 * compared, never dereferenced). Returns JVPATTN_OK or the error code
 * jvpattn_fwd would return. */
int jvpattn_check_fwd(const jvpattn_params* params,
                      const void* q, const void* k, const void* v,
                      const void* tq, const void* tk, const void* tv,
                      const void* mask,
                      const void* o, const void* to, const float* lse, const float* tlse);

/* The forward pass with tangents.
 *   q, tq, o, to : [B, H, Nq, d] contiguous, element type params->dtype
 *   k, v, tk, tv : [B, Hkv, Nk, d] contiguous (Hkv = H unless grouped)
 *   tq, tk, tv   : may each be NULL, meaning a zero tangent
 *   mask         : NULL iff mask_kind == NONE; layout given by the strides
 *   lse, tlse    : [B, H, Nq] float32; tlse may be NULL (not written)
 * Outputs are fully overwritten and must not overlap the inputs or each
 * other. Inputs are read only. Arithmetic: products on the matrix cores in
 * float32 accumulation; softmax statistics in float32; for 16-bit inputs the
 * softmax weights and their products with the score tangent are rounded to
 * the input type before the value products; O and dO are rounded to nearest
 * even. Float32 inputs use float32 matrix products throughout. For float16
 * the rounded products of weights and score tangents stay finite while
 * |dS| < 1024 (weights are kept at most 64 against the running reference). */
int jvpattn_fwd(const jvpattn_params* params,
                const void* q, const void* k, const void* v,
                const void* tq, const void* tk, const void* tv,
                const void* mask,
                void* o, void* to, float* lse, float* tlse,
                void* stream);

/* The forward pass along a tangent of the additive mask as well: the same
 * call as jvpattn_fwd, plus
 *   tmask : the tangent dM of the additive mask, laid out exactly as `mask`
 *           (same strides, element type params->dtype); NULL = zero.
 * The score tangent becomes dS = scale (dQ K^T + Q dK^T) + dM, so dO, tlse
 * are the derivatives of O, lse along (dQ, dK, dV, dM): the additive mask is
 * the float attn_mask input of scaled_dot_product_attention, of which the
 * "JVP Flash Attention" README (section "Usage") makes the method a drop-in.
 * Errors as jvpattn_fwd, and JVPATTN_ERR_MASK if tmask is given without an
 * additive mask, JVPATTN_ERR_ALIGN if it is not aligned to the element size,
 * JVPATTN_ERR_ALIAS if it overlaps an output. jvpattn_bwd differentiates the
 * forward without a mask tangent, jvpattn_bwd_tmask the forward with one. */
int jvpattn_fwd_tmask(const jvpattn_params* params,
                      const void* q, const void* k, const void* v,
                      const void* tq, const void* tk, const void* tv,
                      const void* mask, const void* tmask,
                      void* o, void* to, float* lse, float* tlse,
                      void* stream);

/* Host-only validation of a jvpattn_fwd_tmask call (pointers compared, never
 * dereferenced); returns JVPATTN_OK or the code jvpattn_fwd_tmask would return. */
int jvpattn_check_fwd_tmask(const jvpattn_params* params,
                            const void* q, const void* k, const void* v,
                            const void* tq, const void* tk, const void* tv,
                            const void* mask, const void* tmask,
                            const void* o, const void* to, const float* lse, const float* tlse);

/* ------------------------------------------------------------ reverse pass
 *
 * The pullback of the pair (O, dO) that jvpattn_fwd returns: reverse mode
 * taken over the forward-mode pass, which is how the "JVP Flash Attention"
 * README (section "Description") reaches Hessian-vector products. With
 * cotangents go of O and gto of dO, i.e. for L = <go, O> + <gto, dO>, it
 * returns
 *   dq, dk, dv    = dL/dq, dL/dk, dL/dv
 *   dtq, dtk, dtv = dL/dtq, dL/dtk, dL/dtv   (the cotangents of the tangents)
 * The additive mask is a constant: no gradient is returned for it.
 *
 *   params, q, k, v, tq, tk, tv, mask : exactly as given to jvpattn_fwd
 *   o, to, lse, tlse : what jvpattn_fwd returned for them (all four required)
 *   go, gto          : [B, H, Nq, d], the element type; either may be NULL,
 *                      meaning a zero cotangent
 *   dq, dtq          : [B, H, Nq, d] outputs; dk, dv, dtk, dtv: [B, Hkv, Nk, d]
 *                      (with grouped heads, each sums over its H / Hkv query heads);
 *                      dtq, dtk, dtv may be NULL (not written), e.g. for the
 *                      plain attention backward with gto = NULL
 *   workspace        : device memory of at least
 *                      jvpattn_bwd_workspace_bytes(params) bytes, 256-byte
 *                      aligned, owned by the caller; contents on entry are
 *                      ignored and overwritten (per-row statistics). Calls
 *                      that may run at the same time need separate
 *                      workspaces.
 * Outputs are fully overwritten and must not overlap an input, each other
 * or the workspace. Supported: float16 and bfloat16 with d = 64 or 128,
 * float32 with d = 64 (other element types return JVPATTN_ERR_DTYPE, other
 * d JVPATTN_ERR_HEADDIM, before any work is queued), every mask kind,
 * grouped key/value heads.
 * Arithmetic: products on the matrix cores with float32 accumulation; for
 * 16-bit inputs the recomputed softmax weights, their tangents and the score
 * cotangents are rounded to the input type before the products that consume
 * them (float32: float32 products throughout); results are rounded to
 * nearest even. */

/* Bytes of workspace jvpattn_bwd needs for these parameters, or a negative
 * JVPATTN_ERR_* code if the parameters are invalid for it. */
int64_t jvpattn_bwd_workspace_bytes(const jvpattn_params* params);

/* Host-only validation of a jvpattn_bwd call (pointers compared, never
 * dereferenced); returns JVPATTN_OK or the code jvpattn_bwd would return. */
int jvpattn_check_bwd(const jvpattn_params* params,
                      const void* q, const void* k, const void* v,
                      const void* tq, const void* tk, const void* tv,
                      const void* mask,
                      const void* o, const void* to, const float* lse, const float* tlse,
                      const void* go, const void* gto,
                      const void* dq, const void* dk, const void* dv,
                      const void* dtq, const void* dtk, const void* dtv,
                      const void* workspace, size_t workspace_bytes);

int jvpattn_bwd(const jvpattn_params* params,
                const void* q, const void* k, const void* v,
                const void* tq, const void* tk, const void* tv,
                const void* mask,
                const void* o, const void* to, const float* lse, const float* tlse,
                const void* go, const void* gto,
                void* dq, void* dk, void* dv,
                void* dtq, void* dtk, void* dtv,
                void* workspace, size_t workspace_bytes,
                void* stream);

/* The reverse pass without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, results and errors are those
 * of jvpattn_bwd without `workspace` / `workspace_bytes`: the per-row
 * statistics live instead in a fixed scratch array inside the library, one
 * per GPU, allocated when the library's code is first loaded on that GPU and
 * held until the process ends (4 float32 per query row, 16 MiB). Limits and
 * behaviour:
 *   - B * H * Nq <= JVPATTN_BWD_NOALLOC_MAX_ROWS, else JVPATTN_ERR_SCRATCH
 *     (checked before anything else; nothing is queued);
 *   - the GPU is the one `stream` belongs to (NULL: the current device);
 *   - every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (each entry this call reads, it writes first): calls
 *     that may overlap on one GPU -- concurrent streams, other threads --
 *     race and must be serialised by the caller;
 *   - no memory is allocated or freed by the call.
 * Only the forward without a mask tangent (jvpattn_fwd) is differentiated. */
#define JVPATTN_BWD_NOALLOC_MAX_ROWS (1 << 20)
int jvpattn_bwd_noalloc(const jvpattn_params* params,
                        const void* q, const void* k, const void* v,
                        const void* tq, const void* tk, const void* tv,
                        const void* mask,
                        const void* o, const void* to, const float* lse, const float* tlse,
                        const void* go, const void* gto,
                        void* dq, void* dk, void* dv,
                        void* dtq, void* dtk, void* dtv,
                        void* stream);

/* The reverse pass of the forward taken along a tangent of the additive
 * mask as well (jvpattn_fwd_tmask): the same call as jvpattn_bwd plus
 *   tmask : that tangent dM, laid out exactly as `mask`; NULL = zero.
 * The score tangent it differentiates is dS = scale (dQ K^T + Q dK^T) + dM;
 * the mask and dM are constants of the map (no cotangent is returned for
 * them). Errors as jvpattn_bwd, plus jvpattn_fwd_tmask's for tmask, and
 * JVPATTN_ERR_ALIAS / JVPATTN_ERR_WORKSPACE if it overlaps a gradient or
 * the workspace. For callers that differentiate through a mask tangent. */
int jvpattn_bwd_tmask(const jvpattn_params* params,
                      const void* q, const void* k, const void* v,
                      const void* tq, const void* tk, const void* tv,
                      const void* mask, const void* tmask,
                      const void* o, const void* to, const float* lse, const float* tlse,
                      const void* go, const void* gto,
                      void* dq, void* dk, void* dv,
                      void* dtq, void* dtk, void* dtv,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/* Host-only validation of a jvpattn_bwd_tmask call (pointers compared, never
 * dereferenced); returns JVPATTN_OK or the code jvpattn_bwd_tmask would return. */
int jvpattn_check_bwd_tmask(const jvpattn_params* params,
                            const void* q, const void* k, const void* v,
                            const void* tq, const void* tk, const void* tv,
                            const void* mask, const void* tmask,
                            const void* o, const void* to, const float* lse, const float* tlse,
                            const void* go, const void* gto,
                            const void* dq, const void* dk, const void* dv,
                            const void* dtq, const void* dtk, const void* dtv,
                            const void* workspace, size_t workspace_bytes);

/* ------------------------------------------------------ algorithm selection
 *
 * Kernel families of the 16-bit forward. The library picks one per call from
 * the grid it would launch; these values force one (tuning and testing).
 * Every family computes the same operation to the same rounding rules. */
typedef enum {
  JVPATTN_ALGO_AUTO = -1,
  JVPATTN_FWD_WG4 = 0,       /* 4 waves, 128 query rows per workgroup (every d) */
  JVPATTN_FWD_PINGPONG = 1,  /* 8 waves in two alternating groups, 256 rows (d = 64) */
  JVPATTN_FWD_SPLIT = 2,     /* 4-wave body, key range split over two wave groups (d = 64) */
  JVPATTN_FWD_SPLIT64 = 3    /* the same on 64-row blocks, two waves per group (d = 64) */
} jvpattn_fwd_kernel;

/* Force the forward's launch plan for later jvpattn_fwd / jvpattn_fwd_tmask
 * calls in this process (a process-wide setting; calls already queued are
 * unaffected). Each argument is JVPATTN_ALGO_AUTO (-1) for the library's own
 * choice, or:
 *   kernel    : a jvpattn_fwd_kernel value; a family that does not exist for
 *               a call's type and head dimension falls back to the 4-wave
 *               kernel (float32 always runs its own kernel);
 *   order     : 0 = heaviest query blocks first over all heads, 1 = the query
 *               blocks of each head back to back on one XCD;
 *   key_range : 0 = no mask early-outs: neither the scan of a mask shared by
 *               all query rows for its visible key range, nor the skip of
 *               32 x 32 blocks a mask hides from all 32 rows of a wave
 *               (every block runs); 1 = automatic.
 * Returns JVPATTN_OK, or JVPATTN_ERR_ARG (nothing changed) for a value out of
 * range. Not meant to be changed while another thread launches forwards. */
int jvpattn_fwd_set_algo(int kernel, int order, int key_range);

/* Cap the workgroups of the kernels that walk several blocks per workgroup
 * (with a grid smaller than their count): the mask-free forward kernel for
 * bfloat16 d = 96 / 128 (scale not a power of two) and the mask-free key side
 * of jvpattn_bwd / jvpattn_bwd_noalloc at d = 64. 0 (the default) = what the
 * chip holds at once (one workgroup per CU, rounded down to a multiple of 8);
 * n > 0 = at most n (rounded down to a multiple of 8 when n >= 8). Results do
 * not depend on it. A process-wide setting for later calls, like
 * jvpattn_fwd_set_algo; for tests and tuning. Returns JVPATTN_OK, or
 * JVPATTN_ERR_ARG for n < 0. */
int jvpattn_set_workgroups(int max_workgroups);

/* How jvpattn_bwd / jvpattn_bwd_tmask queue their key-side and query-side
 * kernels, which depend only on the per-row statistics both read:
 *   0 : one after the other on the caller's stream;
 *   1 : the query side on a second stream of the library's (one per device,
 *       created with two events on the first such call and kept until the
 *       process ends), which waits for the statistics on the caller's stream;
 *       the caller's stream then waits for the query side, so work queued on
 *       it afterwards sees every gradient, as in mode 0. The query side's
 *       workgroups take the compute units the key side's release;
 *  -1 : (the default) mode 1 where the key side alone would leave compute
 *       units idle -- fewer key-side items (128-key blocks times key/value
 *       heads) than CUs, or with causal set fewer than two per CU -- and for
 *       d = 128; else mode 0.
 * A call whose stream is being captured into a graph, and every
 * jvpattn_bwd_noalloc call, uses mode 0. Results do not depend on the mode.
 * Process-wide, for later calls. Returns JVPATTN_OK, or JVPATTN_ERR_ARG for
 * another value. */
int jvpattn_bwd_set_overlap(int mode);

/* A static, human-readable description of a return code. */
const char* jvpattn_strerror(int code);

/* The HIP error code (hipError_t value) of the most recent JVPATTN_ERR_HIP
 * on the calling thread, or 0. */
int jvpattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JVPATTN_H */
