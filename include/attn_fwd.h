/*
 * attn_fwd.h - C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is attention forward written as a stream of tiles:
 *   S = Q·Kᵀ·scale, an optional causal mask, a row softmax done online across
 *   K/V tiles (exp -> sum -> divide), O = P·V, plus the per-row logsumexp.
 * Sources: "CS149 L11: Programming Specialized Hardware" (quidproquo.cc),
 * section 5 (slide 48: softmax as Map(exp) -> Reduce(+) -> Zip(/); slide 54:
 * FlashAttention as the chain Q·Kᵀ, Mask, Softmax, Dropout, ×V) and section 6
 * (the decoder's Q·Kᵀ, scale, mask, softmax, ×V); "Distilling a 4.5 hour CUDA
 * talk" (levidiamode.com), section 7 (Q resident, K/V streamed through on-chip
 * memory, running max and normalizer).
 *
 * Conventions shared by every entry point:
 *   - Tensors are 4-D [B, H, N, d] with the innermost (d) stride 1. Their
 *     (b, h, n) strides are given in elements; a zero stride triple means
 *     "contiguous". Every stride and every base pointer must be 16-byte
 *     aligned (a multiple of 8 elements for bf16, 4 for fp32).
 *   - Q is [B, H_q, N, d], K is [B, H_kv, N_kv, d], V is [B, H_kv, N_kv, d_v],
 *     O is [B, H_q, N, d_v]; logsumexp is [B, H_q, N] fp32, contiguous.
 *     Query head h reads K/V head h / (H_q / H_kv) (contiguous GQA groups).
 *   - causal masks key j for query row i when j > i (top-left alignment) and
 *     needs N_kv == N. Dropout is not applied (probability 0).
 *   - logsumexp[b,h,i] = ln(sum_j exp(scale * q_i·k_j)) over unmasked keys.
 *   - All device buffers are owned by the caller, who keeps them alive until
 *     the work queued on the stream has finished. The library allocates no
 *     device memory; its only device memory of its own is the static scratch
 *     of attn_fwd_run_split_noalloc, part of the loaded code object.
 *   - Every function returns a status code; nothing throws or aborts across
 *     the ABI.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_fwd_plan attn_fwd_plan; /* opaque, host-side, immutable */

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* malformed argument (sizes, strides, pointers) */
    ATTN_ERR_UNSUPPORTED = 2, /* well-formed but no kernel variant serves it */
    ATTN_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
    ATTN_ERR_NOMEM = 4,       /* host allocation of the plan failed */
    ATTN_ERR_TOO_LARGE = 5    /* the problem needs more scratch than the library's
                                 static buffer holds (attn_fwd_run_split_noalloc) */
} attn_status;

typedef enum {
    ATTN_BF16 = 0, /* Q, K, V and O in bf16 */
    ATTN_FP32 = 1  /* Q, K, V and O in fp32; the tiles are rounded to bf16
                      (round-to-nearest-even) before the MFMA contractions */
} attn_dtype;

typedef struct {
    int64_t B, H_q, H_kv;
    int64_t N;        /* query rows per head (N_q) */
    int64_t d;        /* head dimension of Q and K (d_qk) */
    int64_t N_kv;     /* key/value rows per head; 0 means N */
    int64_t d_v;      /* head dimension of V and O; 0 means d */
    int32_t causal;   /* 0 or 1 */
    float scale;      /* softmax scale, finite and > 0 (e.g. 1/sqrt(d)) */
    int32_t dtype;    /* attn_dtype */
    int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3]; /* (b,h,n) */
} attn_fwd_params;

/*
 * attn_fwd_create - validate a problem and choose its kernel variant.
 * Arguments are the problem of the whole library: B, H_q, H_kv, N, d, causal
 * and scale, with bf16 tensors, contiguous [B, H, N, d] layout, N_kv = N and
 * d_v = d. On success *plan receives a new plan (free it with
 * attn_fwd_destroy). Makes no HIP call. Returns ATTN_ERR_INVALID for
 * non-positive sizes, H_q not a multiple of H_kv, a non-finite or
 * non-positive scale, or plan == NULL; ATTN_ERR_UNSUPPORTED for head
 * dimensions without a kernel (here d = 64 and d = 128; attn_fwd_create_ex
 * also takes d = 576 with d_v = 512).
 */
attn_status attn_fwd_create(attn_fwd_plan **plan, int64_t B, int64_t H_q, int64_t H_kv,
                            int64_t N, int64_t d, int32_t causal, float scale);

/*
 * attn_fwd_create_ex - as attn_fwd_create, from a full descriptor: adds N_kv,
 * d_v, the dtype and explicit strides. Extra ATTN_ERR_INVALID cases: causal
 * with N_kv != N, strides that are not 16-byte multiples, row strides below
 * the row width, or a tensor whose [N, d] slab exceeds 2^31 elements.
 * Supported (d, d_v, dtype): (64, 64, bf16), (128, 128, bf16),
 * (64, 64, fp32), (576, 512, bf16).
 */
attn_status attn_fwd_create_ex(const attn_fwd_params *params, attn_fwd_plan **plan);

/*
 * attn_fwd_run - queue the attention forward pass on `stream` (a hipStream_t;
 * NULL is the default stream). Q, K, V, O are device pointers with the plan's
 * dtype and strides; lse is a device pointer to B*H_q*N floats, or NULL to
 * skip writing logsumexp. V may alias K (e.g. V = the first d_v columns of K
 * through its strides). Returns immediately; never synchronizes. Returns
 * ATTN_ERR_INVALID for a NULL plan or tensor pointer or a pointer that is not
 * 16-byte aligned (checked before any HIP call), ATTN_ERR_HIP if the launch
 * fails.
 */
attn_status attn_fwd_run(const attn_fwd_plan *plan, const void *Q, const void *K,
                         const void *V, void *O, float *lse, void *stream);

/*
 * attn_fwd_run_dropout - attn_fwd_run with dropout between the softmax and
 * the product with V ("CS149 L11: Programming Specialized Hardware", section
 * 5, slide 54: Q·Kᵀ, Mask, Softmax, Dropout, ×V). Every probability p_ij is
 * replaced by p_ij * keep_ij / (1 - q) with q = floor(256 * p_drop) / 256
 * (the drop probability is taken in steps of 1/256); logsumexp stays that of
 * the softmax before dropout. keep_ij = [byte_ij >= 256 q], where byte_ij is
 * one byte of the counter-based generator Philox4x32-10 (Salmon et al.,
 * SC'11) with key (seed mod 2^32, seed / 2^32), counter
 * (i, 2 (j / 32) + (j / 4) mod 2, b H_q + h, 0), output word (j / 8) mod 4,
 * byte j mod 4 - so the mask depends only on (seed, b, h, i, j) and is the
 * same for any launch configuration.
 * p_drop must be in [0, 1) (ATTN_ERR_INVALID otherwise, also for NaN);
 * q == 0 runs attn_fwd_run. Served for d = 64 and d = 128 (bf16, and fp32 at
 * d = 64); the wide-head variant returns ATTN_ERR_UNSUPPORTED. Pointers,
 * alignment and stream as for attn_fwd_run.
 */
attn_status attn_fwd_run_dropout(const attn_fwd_plan *plan, const void *Q, const void *K,
                                 const void *V, void *O, float *lse, float p_drop,
                                 uint64_t seed, void *stream);

/*
 * attn_rope_bf16 - rotary position embedding of a [B, H, N, d] bf16 tensor
 * (the step before attention in the decoder chain of "CS149 L11: Programming
 * Specialized Hardware", section 6; the pages' load-compute-store-finish
 * example, "Distilling a 4.5 hour CUDA talk", section 12). Reading (the pages
 * do not write the formula): the RoFormer rotation of interleaved pairs,
 * pair k of the row at position n (its index) turned by
 * theta = n * base^(-2k / d):
 *   Y[2k] = X[2k] cos theta - X[2k+1] sin theta,
 *   Y[2k+1] = X[2k] sin theta + X[2k+1] cos theta,
 * in fp32 (the angle reduced in fp64), rounded to bf16.
 * X, Y: device pointers, 16-byte aligned, (b, h, n) strides in elements as
 * for attention (NULL or all-zero = contiguous), multiples of 8. Y may be X.
 * d % 8 == 0, base finite and > 1 (else ATTN_ERR_INVALID); an empty tensor
 * queues nothing. Asynchronous on `stream`.
 */
attn_status attn_rope_bf16(const void *X, void *Y, int64_t B, int64_t H, int64_t N, int64_t d,
                           const int64_t x_strides[3], const int64_t y_strides[3], float base,
                           void *stream);

/*
 * attn_fwd_rope_workspace_bytes - bytes of the workspace attn_fwd_run_rope
 * needs for this plan (B * H_kv * N_kv * d bf16), or -1 if the plan's variant
 * has no RoPE path (only bf16 with d = 64 or 128 has one).
 */
int64_t attn_fwd_rope_workspace_bytes(const attn_fwd_plan *plan);

/*
 * attn_fwd_run_rope - attention of RoPE(Q) and RoPE(K) (positions = row
 * indices, as attn_rope_bf16 with `base`) against V. Q is rotated in
 * registers as the kernel loads it; K is rotated once per kv head into the
 * caller's workspace k_rot (k_rot_bytes >= attn_fwd_rope_workspace_bytes;
 * 16-byte aligned; it may be K itself, which is then rotated in place, but
 * must not overlap Q, V or O) and the kernel reads K from there. O and logsumexp as for attn_fwd_run.
 * ATTN_ERR_UNSUPPORTED for plans without a RoPE path; ATTN_ERR_INVALID for
 * NULL or misaligned pointers, a short workspace or a bad base.
 */
attn_status attn_fwd_run_rope(const attn_fwd_plan *plan, const void *Q, const void *K,
                              const void *V, void *O, float *lse, float base, void *k_rot,
                              int64_t k_rot_bytes, void *stream);

/*
 * Split-KV forward (few query rows per kv head, long key sequences: decode).
 * The keys of each kv head are cut into n_splits contiguous ranges; each
 * range's attention of all the group's query rows is computed separately and
 * written, as O / l (fp32) and its logsumexp, to a caller-provided workspace;
 * a second kernel merges the ranges exactly: lse = ln Σ_s exp(lse_s),
 * O = Σ_s exp(lse_s - lse) O_s. The result equals attn_fwd_run's (same
 * method, "Distilling a 4.5 hour CUDA talk", section 7: the running max and
 * normalizer carried across key tiles, here also across ranges).
 * Served problems, never causal:
 *   - (d, d_v, dtype) (64, 64, bf16) or (128, 128, bf16) with
 *     (H_q / H_kv) * N <= 64 (all query rows of a kv head fit one
 *     workgroup) and B * H_kv <= 2^18 (the launches' work-items fit 32 bits);
 *   - (576, 512, bf16), wide heads whose V is the first 512 columns of K
 *     (V == K with K's strides: the kernel reads V from the K tiles it
 *     copies), any N: each workgroup takes 64 query rows of one (batch,
 *     head) over one key range, with B * H_q * ceil(N / 64) < 2^17 (the
 *     launch's work-items fit 32 bits at 64 ranges).
 *     Whether V lies inside K is known only from the pointers, so
 *     attn_fwd_split_count serves such plans and the run entry points return
 *     ATTN_ERR_UNSUPPORTED, before any HIP call, for a V of its own
 *     (attn_fwd_run serves that).
 */

/*
 * attn_fwd_split_count - the number of key ranges the library would use for
 * the plan (enough workgroups for every CU, at most 64, at least one key tile
 * each: 64 keys, 32 for wide heads), or 0 if the split path does not serve
 * the plan (or plan is NULL).
 */
int32_t attn_fwd_split_count(const attn_fwd_plan *plan);

/*
 * attn_fwd_split_workspace_bytes - device bytes attn_fwd_run_split needs for
 * n_splits key ranges (n_splits <= 0: the library's count):
 * n_splits * B * H_q * N * (d_v + 1) * 4. Returns -1 if the split path does
 * not serve the plan or n_splits > 64.
 */
int64_t attn_fwd_split_workspace_bytes(const attn_fwd_plan *plan, int32_t n_splits);

/*
 * attn_fwd_run_split - as attn_fwd_run, through n_splits key ranges
 * (n_splits <= 0: the library's count). workspace is a caller-owned device
 * buffer of at least attn_fwd_split_workspace_bytes(plan, n_splits) bytes,
 * 16-byte aligned; its contents on entry do not matter and on return are
 * scratch. Two kernels are queued on `stream`; calls that share a workspace
 * must not overlap. Returns ATTN_ERR_INVALID for NULL or misaligned pointers,
 * n_splits > 64 or a short workspace; ATTN_ERR_UNSUPPORTED if the split path
 * does not serve the plan or (wide heads) V is not inside K; ATTN_ERR_HIP if
 * a launch fails.
 */
attn_status attn_fwd_run_split(const attn_fwd_plan *plan, const void *Q, const void *K,
                               const void *V, void *O, float *lse, int32_t n_splits,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_run_split_noalloc - attn_fwd_run_split for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The per-range partial results go to a
 * buffer the library keeps in static device memory, ATTN_SPLIT_SCRATCH_BYTES
 * (16 MiB) per GPU, held by every GPU the library runs on until the process
 * ends, instead of a caller workspace. Nothing is allocated: no hipMalloc,
 * hipFree or allocating library routine. The first call on a device looks
 * the buffer's address up on that device (the stream's device, or the
 * current device for the NULL stream); later calls reuse it.
 * Arguments as attn_fwd_run_split without the workspace. Returns
 * ATTN_ERR_TOO_LARGE (before any HIP call) when
 * attn_fwd_split_workspace_bytes(plan, n_splits) exceeds
 * ATTN_SPLIT_SCRATCH_BYTES; the other argument errors as attn_fwd_run_split;
 * ATTN_ERR_HIP when the buffer's address cannot be found or a launch fails.
 * Every call on a GPU shares that GPU's buffer, which keeps the last call's
 * contents (nothing in it needs clearing between calls): calls that overlap
 * on one GPU - on other streams or from other threads - race, and the
 * caller must order them.
 */
#define ATTN_SPLIT_SCRATCH_BYTES (16ll * 1024 * 1024)
attn_status attn_fwd_run_split_noalloc(const attn_fwd_plan *plan, const void *Q, const void *K,
                                       const void *V, void *O, float *lse, int32_t n_splits,
                                       void *stream);

/* attn_fwd_destroy - free a plan. NULL is accepted and ignored. */
void attn_fwd_destroy(attn_fwd_plan *plan);

/* attn_status_str - a static, human-readable name for a status code. */
const char *attn_status_str(attn_status status);

/*
 * attn_fwd_plan_info - launch geometry chosen by a plan, for tests and
 * reports: work items (one per batch, query head and query tile; one
 * workgroup each, or, where they fill whole rounds of the 256 CUs and the kv
 * heads split evenly over the 8 XCDs, 256 persistent workgroups taking them
 * in turn), threads per workgroup, query rows and key rows per tile, and LDS
 * bytes per workgroup. Any output pointer may be NULL.
 */
attn_status attn_fwd_plan_info(const attn_fwd_plan *plan, int64_t *grid, int32_t *block,
                               int32_t *tile_q, int32_t *tile_k, int32_t *lds_bytes);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
