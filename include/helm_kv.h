/*
 * helm_kv.h — C ABI of the MI355X (gfx950) cross-model KV-cache transfer.
 *
 * The operation (pages: "Helm Intelligent Routing", section "Why carrying the
 * cache across is the hard part"; the Qwen3 cache-mapping write-up, section
 * "A linear bridge, strangely enough, suffices", its fit/map listing and its
 * strip-RoPE / map / apply-RoPE diagram).  For every target layer l < L_t,
 * KV head h < H and token t < T, with half = D/2 and the rotate-half RoPE
 * rotation R(p; theta) that turns pair (i, i+half) by p * theta^(-2i/D):
 *
 *   x_k = concat_{j<k} R(-src_pos[t]; theta_src) src_k[layer_sel[l,j], h, t, :]
 *   x_v = concat_{j<k} src_v[layer_sel[l,j], h, t, :]
 *   out_k[l, h, t, :] = R(+tgt_pos[t]; theta_tgt) (x_k · W_k[l, h] + b_k[l, h])
 *   out_v[l, h, t, :] =                            x_v · W_v[l, h] + b_v[l, h]
 *
 * i.e. un-rotate the pilot's keys into content space at their source
 * positions, gather the same KV head from the k selected source layers (in
 * the order of the layer_sel row), apply the per-(target layer, head) affine
 * map — one for keys, one for values, W stored in-major [k*D][D] as in the
 * listing's x @ w + b — and re-rotate the mapped keys at the positions they
 * take in the target sequence.  The re-rotation is always applied; there is
 * no switch to skip it.
 *
 * Precision.  bf16 storage: the un-rotated key is formed in fp32 and rounded
 * once (nearest-even) to bf16 as the operand of a bf16 x bf16 matrix-core
 * product with fp32 accumulation; bias and forward rotation are fp32; the
 * result is rounded once (nearest-even) to bf16.  fp32 storage: the whole
 * path is fp32.  RoPE angles are formed in fp64 (p * w_i) and their cos/sin
 * rounded once to fp32, so positions up to 2^31 keep full accuracy.
 *
 * Pair requirements ("Helm Intelligent Routing", section "Requirements"):
 * source and target share the KV-head count H and the head dimension D;
 * their layer counts may differ.
 *
 * Conventions for every entry point.
 *   - Every pointer to tensor data is a DEVICE pointer owned by the caller
 *     (e.g. a torch tensor's data_ptr()); the library never frees, keeps or
 *     allocates memory.  Tensors are dense, row-major, in the layouts given.
 *   - Calls are asynchronous on shape->stream (a hipStream_t; NULL = the
 *     null stream).  A HELM_OK return means the work was enqueued; device
 *     faults surface at the caller's next synchronisation.
 *   - All validation happens on the host before anything is enqueued: a call
 *     that returns an error has written nothing, so the caller can fall back
 *     to a normal target prefill ("Helm Intelligent Routing", section "What
 *     happens when a transfer cannot be used": a refused transfer never fails
 *     a request).  helm_last_error() then names the specific reason.
 *   - Device-side tables (layer_sel, block tables, cu_seqlens) are not read
 *     by the host.  Check them once with helm_mapper_check /
 *     helm_paged_check on host copies.  The kernels still bounds-check every
 *     index they read: a target layer whose layer_sel row holds an index
 *     outside [0, L_s), or a token whose block id lies outside its pool, is
 *     left unwritten instead of reading or writing out of bounds.
 *   - Thread safety: calls may be made from several host threads; the only
 *     library state is a per-thread error string and a per-device cache of
 *     the device check.
 */
#ifndef HELM_KV_H
#define HELM_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HELM_ABI_VERSION 1

/* Status codes.  HELM_E_NO_DEVICE is 4 like the calibration tool's "no
 * accelerator on this host" exit code ("Helm Intelligent Routing", section
 * "What calibration does, and what it costs"). */
typedef enum {
  HELM_OK = 0,
  HELM_E_INVALID_ARG = 1,  /* null pointer, non-positive size, k outside 1..L_s, overflow */
  HELM_E_PAIR_SHAPE = 2,   /* D odd or unsupported for the dtype */
  HELM_E_LAYER_SEL = 3,    /* a layer_sel entry outside [0, L_s) (helm_mapper_check) */
  HELM_E_NO_DEVICE = 4,    /* no GPU visible */
  HELM_E_DTYPE = 5,        /* unknown dtype code */
  HELM_E_ARCH = 6,         /* the current device is not gfx950 */
  HELM_E_WORKSPACE = 7,    /* workspace missing, misaligned or too small */
  HELM_E_ALIAS = 8,        /* an output byte range overlaps an input or the other output */
  HELM_E_PAGED_TABLE = 9,  /* bad cu_seqlens or block table (helm_paged_check) */
  HELM_E_LAUNCH = 10       /* a HIP call failed; helm_last_error() holds its text */
} helm_status_t;

/* Storage dtype of caches and maps.  Biases are always fp32. */
typedef enum { HELM_BF16 = 0, HELM_F32 = 1 } helm_dtype_t;

/* Supported head dimensions: D = 64 or 128 (both dtypes). */

/* Contiguous transfer shape.
 *   src_k, src_v : [L_s, H, T, D]      dtype; keys stored rotated at src_pos
 *   src_pos      : [T]                 int32, any values (negative allowed)
 *   tgt_pos      : [T]                 int32, positions in the target sequence
 *   layer_sel    : [L_t, k]            int32 in [0, L_s); duplicates allowed
 *   W_k, W_v     : [L_t, H, k*D, D]    dtype, in-major (row m = input feature)
 *   b_k, b_v     : [L_t, H, D]         fp32
 *   out_k, out_v : [L_t, H, T, D]      dtype; fully overwritten
 * Workspace: device memory of at least helm_kv_workspace_bytes(shape)
 * bytes, 256-byte aligned, not shared with a concurrent call. */
typedef struct {
  int32_t n_src_layers;    /* L_s >= 1 */
  int32_t n_tgt_layers;    /* L_t >= 1 */
  int32_t n_kv_heads;      /* H >= 1 */
  int32_t head_dim;        /* D in {64, 128} */
  int32_t k;               /* 1 <= k <= L_s */
  int32_t dtype;           /* helm_dtype_t */
  int64_t n_tokens;        /* T >= 0; T = 0 returns HELM_OK without touching
                              any pointer or the device */
  double rope_theta_src;   /* > 0; the pilot's RoPE base */
  double rope_theta_tgt;   /* > 0; the target's RoPE base */
  void* stream;            /* hipStream_t */
  void* workspace;         /* device scratch */
  size_t workspace_bytes;
} helm_shape_t;

/* Paged transfer shape.  Pools are per-layer paged caches with pages of
 * block_size token slots (16 in the benchmarked workload):
 *   src_k_pool, src_v_pool : [L_s, n_src_blocks, block_size, H, D] dtype
 *   tgt_k_pool, tgt_v_pool : [L_t, n_tgt_blocks, block_size, H, D] dtype
 *   src_block_table        : [R, max_blocks_src] int32
 *   tgt_block_table        : [R, max_blocks_tgt] int32
 *   cu_seqlens             : [R+1] int32, cu[0] = 0, non-decreasing,
 *                            cu[R] = n_tokens_total
 *   src_pos, tgt_pos       : [n_tokens_total] int32 over packed tokens
 * Token t of request r (packed index cu[r] + t) is read from slot
 * t % block_size of block src_block_table[r][t / block_size] of every
 * selected source layer and written to slot t % block_size of block
 * tgt_block_table[r][t / block_size] of every target layer.  No other slot
 * of the target pools is touched.  Two tokens must never share a target
 * slot (helm_paged_check tests that the used target entries are distinct). */
typedef struct {
  int32_t n_src_layers, n_tgt_layers, n_kv_heads, head_dim, k, dtype;
  int32_t block_size;      /* >= 1 */
  int32_t n_requests;      /* R >= 1 */
  int32_t max_blocks_src;  /* row stride of src_block_table */
  int32_t max_blocks_tgt;  /* row stride of tgt_block_table */
  int32_t n_src_blocks;    /* blocks per source pool layer */
  int32_t n_tgt_blocks;    /* blocks per target pool layer */
  int64_t n_tokens_total;  /* cu_seqlens[R]; the host passes it (no device read);
                              0 returns HELM_OK without touching anything */
  double rope_theta_src, rope_theta_tgt;
  void* stream;
  void* workspace;
  size_t workspace_bytes;
} helm_paged_shape_t;

/* The contiguous transfer (definition at the top of this file).
 * Returns HELM_OK once the kernels are enqueued on shape->stream, or an
 * error with nothing enqueued.  out_k / out_v must not overlap any input. */
int helm_kv_transfer(const void* src_k, const void* src_v,
                     const int32_t* src_pos, const int32_t* tgt_pos,
                     const int32_t* layer_sel,
                     const void* W_k, const float* b_k,
                     const void* W_v, const float* b_v,
                     void* out_k, void* out_v,
                     const helm_shape_t* shape);

/* helm_kv_transfer in two separately enqueued stages, for callers that map
 * several batches of caches at the same positions, and for timing the map
 * alone.  stages is a bit mask:
 *   HELM_STAGE_TABLES (1)  write the RoPE (cos, sin) tables of src_pos /
 *                          tgt_pos into shape->workspace;
 *   HELM_STAGE_MAP    (2)  run the map, reading the tables already in the
 *                          workspace: they must come from an earlier call
 *                          with HELM_STAGE_TABLES (or helm_kv_transfer) on
 *                          the same positions, thetas, n_tokens and
 *                          head_dim, ordered before this one.  The library
 *                          does not check that; stale tables give wrong keys.
 *   HELM_STAGE_ALL    (3)  both, exactly helm_kv_transfer.
 * Every pointer and shape check of helm_kv_transfer applies in every stage;
 * same return convention. */
#define HELM_STAGE_TABLES 1
#define HELM_STAGE_MAP 2
#define HELM_STAGE_ALL 3
int helm_kv_transfer_stage(int stages,
                           const void* src_k, const void* src_v,
                           const int32_t* src_pos, const int32_t* tgt_pos,
                           const int32_t* layer_sel,
                           const void* W_k, const float* b_k,
                           const void* W_v, const float* b_v,
                           void* out_k, void* out_v,
                           const helm_shape_t* shape);

/* helm_kv_transfer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, checks and results as helm_kv_transfer
 * (bit-identical outputs); shape->workspace and workspace_bytes are ignored:
 * the RoPE tables go to a static device buffer of
 * helm_kv_noalloc_max_bytes() bytes (64 MiB) that the library holds on each
 * GPU it runs on until the process ends.  Nothing is allocated or freed.
 * Limit: n_tokens <= 65,536 at head_dim 128 (131,072 at 64); larger calls
 * return HELM_E_WORKSPACE with nothing enqueued.  Every call on one GPU
 * shares that GPU's buffer: calls that overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller; calls in
 * stream order on one stream are safe.  The buffer needs no clearing (each
 * call writes the tables it reads). */
size_t helm_kv_noalloc_max_bytes(void);
int helm_kv_transfer_noalloc(const void* src_k, const void* src_v,
                             const int32_t* src_pos, const int32_t* tgt_pos,
                             const int32_t* layer_sel,
                             const void* W_k, const float* b_k,
                             const void* W_v, const float* b_v,
                             void* out_k, void* out_v,
                             const helm_shape_t* shape);

/* The same transfer on paged caches driven by block tables (knlp "Routing"
 * page, request-flow figure: the selection is applied to the block table and
 * only the selected blocks are written into the paged cache; "Helm
 * Intelligent Routing", section "Current limitation": the installer writes
 * into the inference engine's paged cache).  Same return convention. */
int helm_kv_transfer_paged(const void* src_k_pool, const void* src_v_pool,
                           const int32_t* src_block_table, const int32_t* tgt_block_table,
                           const int32_t* cu_seqlens,
                           const int32_t* src_pos, const int32_t* tgt_pos,
                           const int32_t* layer_sel,
                           const void* W_k, const float* b_k,
                           const void* W_v, const float* b_v,
                           void* tgt_k_pool, void* tgt_v_pool,
                           const helm_paged_shape_t* shape);

/* The wide-input map (the Qwen3 cache-mapping write-up, section "A linear
 * bridge, strangely enough, suffices": the full mapper's x concatenates the
 * KV features of all selected source layers, with one fit per target head
 * for keys and one for values).  Per target layer l and token t:
 *   x[((j*2 + kv)*H + g)*D + d] = kv == 0 ? (R(-src_pos[t]) src_k[sel_j, g, t, :])[d]
 *                                         : src_v[sel_j, g, t, d]
 * (j in layer_sel row order, keys before values, source head g; IN =
 * k*2*H*D features), and for every target head h
 *   out_k[l, h, t, :] = R(+tgt_pos[t]) (x W_k[l, h] + b_k[l, h])
 *   out_v[l, h, t, :] = x W_v[l, h] + b_v[l, h].
 * The un-rotated key is rounded once to bf16 (the map's operand type), as in
 * helm_kv_transfer.  Same arguments and conventions as helm_kv_transfer,
 * except:
 *   W_k, W_v : [L_t, H, IN, D] bf16 (in-major)
 *   dtype    : HELM_BF16 only (HELM_E_DTYPE otherwise); head_dim 128 only
 *              (HELM_E_PAIR_SHAPE otherwise); src_k, src_v, out_k and out_v
 *              16-byte aligned (HELM_E_INVALID_ARG otherwise); W_k and W_v
 *              need only their elements' alignment (16-byte aligned maps are
 *              transposed with 16-byte accesses, others with 2-byte ones)
 *   workspace: helm_kv_wide_workspace_bytes(shape) bytes, 256-byte aligned;
 *              it holds the RoPE tables, the un-rotated source keys
 *              [L_s, H, T, D] and both maps transposed [L_t, H, D, IN]
 *              (40 -> 64 layers, 8 heads, IN = 8192, 32,768 tokens: 4.9 GB).
 * n_tokens = 0 enqueues nothing. */
size_t helm_kv_wide_workspace_bytes(const helm_shape_t* shape);
int helm_kv_transfer_wide(const void* src_k, const void* src_v,
                          const int32_t* src_pos, const int32_t* tgt_pos,
                          const int32_t* layer_sel,
                          const void* W_k, const float* b_k,
                          const void* W_v, const float* b_v,
                          void* out_k, void* out_v,
                          const helm_shape_t* shape);

/* helm_kv_transfer_wide in two separately enqueued stages (for mapping
 * several caches with the same maps and positions, and for timing the
 * product alone).  stages is a bit mask:
 *   HELM_STAGE_TABLES (1)  the preparation: the RoPE tables, the un-rotated
 *                          source keys and both transposed maps, all into
 *                          shape->workspace;
 *   HELM_STAGE_MAP    (2)  the product and its bias / RoPE epilogue, reading
 *                          the workspace: it must hold the preparation of
 *                          the same src_k, positions, thetas, maps and shape,
 *                          ordered before this call (not checked; a stale
 *                          workspace gives wrong outputs);
 *   HELM_STAGE_ALL    (3)  both, exactly helm_kv_transfer_wide.
 * Every check of helm_kv_transfer_wide applies in every stage; stages
 * outside 1..3 give HELM_E_INVALID_ARG. */
int helm_kv_transfer_wide_stage(int stages,
                                const void* src_k, const void* src_v,
                                const int32_t* src_pos, const int32_t* tgt_pos,
                                const int32_t* layer_sel,
                                const void* W_k, const float* b_k,
                                const void* W_v, const float* b_v,
                                void* out_k, void* out_v,
                                const helm_shape_t* shape);

/* KV-cosine diagnostic ("Helm Intelligent Routing", the retention / KL /
 * KV-cosine table: how close the mapped cache is to the target model's
 * own; a low cosine with low retention means the map is wrong).  For every
 * target layer l and head h, and for keys and for values, the cosine of the
 * two [T, D] slabs taken as flat vectors:
 *   cos_out[kv][l][h] = sum(a*b) / (sqrt(sum(a*a)) * sqrt(sum(b*b)))
 * with a from the mapped cache (k_mapped / v_mapped, e.g. out_k / out_v of
 * helm_kv_transfer) and b from the reference cache (k_ref / v_ref, e.g. the
 * target model's own prefill), kv = 0 for keys and 1 for values.  A slab of
 * zeros gives NaN (0/0); with n_tokens = 0 every entry is NaN.
 *   caches : [L_t, H, T, D] contiguous, shape->dtype, device memory
 *   cos_out: [2, L_t, H] float32, device memory, caller-owned; must not
 *            overlap a cache
 * Uses shape->n_tgt_layers, n_kv_heads, n_tokens, head_dim, dtype and stream
 * (the other fields must still pass the transfer's checks; no workspace).
 * Sums are accumulated in fp64 (fp32 within each 16-byte piece).  Enqueued
 * asynchronously on shape->stream; same return convention as
 * helm_kv_transfer (nothing enqueued on an error). */
int helm_kv_cosine(const void* k_mapped, const void* v_mapped,
                   const void* k_ref, const void* v_ref,
                   float* cos_out, const helm_shape_t* shape);

/* Ridge fit of the maps (the Qwen3 cache-mapping write-up, section "A
 * linear bridge, strangely enough, suffices": each target head's key map
 * and value map are fitted separately by ridge regression on centred data,
 * lambda = 0.01, the bias from the means).  For each of n_groups
 * independent groups g (one (target layer, head, K|V) map each), with
 * observations X[g] [N, IN] and targets Y[g] [N, D]:
 *   W[g] = (Xc^T Xc + lambda I)^-1 Xc^T Yc,   b[g] = mean(Y[g]) - mean(X[g]) W[g]
 * (Xc, Yc = the data minus its column means).  Each feature is first
 * shifted by a value taken from the group's first observations: its first
 * value when its first min(N, 64) values share one sign and lie within a
 * factor 1.5 of each other, else 0 (a mean large against the spread would
 * otherwise cost about (mean / spread)^2 * 2^-24 of relative accuracy in
 * the centring of fp32 sums).  The products of the shifted data (each
 * difference exact in bf16 when within a factor 2 of its shift, else
 * rounded to bf16 once) are accumulated in fp32 on the matrix cores, the
 * column sums in fp32 on the vector ALU; the centring, lambda, the Cholesky
 * solve and b (with the means = shifts + sums / N) are fp64; W and b are
 * stored as fp32.
 *   X : [n_groups, n_obs, in_features] bf16, device, 16-byte aligned
 *   Y : [n_groups, n_obs, out_features] bf16, device, 16-byte aligned
 *   W : [n_groups, in_features, out_features] fp32 (in-major, the layout of
 *       the transfer's maps), caller-owned
 *   b : [n_groups, out_features] fp32, caller-owned
 * Limits: dtype HELM_BF16 (HELM_E_DTYPE otherwise); out_features 128 and
 * in_features a multiple of 128 up to 1024 (HELM_E_PAIR_SHAPE otherwise);
 * n_obs >= 1 with n_obs * in_features * 2 below 4 GB; lambda >= 0.  A group
 * whose normal matrix is not positive definite (possible only with
 * lambda = 0) gets NaN in its W and b.  Enqueued on shape->stream; nothing
 * is enqueued on an error; W, b and the workspace must not overlap X, Y or
 * each other (HELM_E_ALIAS). */
typedef struct {
  int64_t n_groups;        /* G >= 1 */
  int64_t n_obs;           /* N >= 1 observations per group */
  int32_t in_features;     /* IN */
  int32_t out_features;    /* D */
  int32_t dtype;           /* helm_dtype_t of X and Y */
  double lambda;           /* ridge penalty, >= 0 (0.01 on the pages) */
  void* stream;            /* hipStream_t */
  void* workspace;         /* device scratch, 256-byte aligned */
  size_t workspace_bytes;
} helm_ridge_shape_t;
/* Workspace bytes of a fit (0 on an invalid shape): the fp32 products
 * [G, IN, IN] and [G, IN, D], the sums and the shifts [G, IN + D] each and
 * the fp64 solve matrix [G, IN, IN + D] (1,024 groups of IN = 512: 4.2 GB). */
size_t helm_ridge_workspace_bytes(const helm_ridge_shape_t* shape);
int helm_ridge_fit(const void* X, const void* Y, float* W, float* b, const helm_ridge_shape_t* shape);
/* The fit in two separately enqueued stages: HELM_STAGE_TABLES (1) the
 * products and sums into the workspace, HELM_STAGE_MAP (2) the solve
 * reading them (the workspace must hold the first stage's results of the
 * same X, Y and shape, ordered before; not checked), HELM_STAGE_ALL (3)
 * both.  For timing the stages alone; same checks and return convention. */
int helm_ridge_fit_stage(int stages, const void* X, const void* Y, float* W, float* b,
                         const helm_ridge_shape_t* shape);

/* Workspace bytes the call with this shape needs (0 on an invalid shape;
 * helm_last_error() then says why).  Pure host arithmetic.  The workspace
 * holds what the transfer derives from the positions — the (cos, sin)
 * tables of the source and target RoPE angles ("Helm Intelligent Routing",
 * section "Why carrying the cache across is the hard part": keys are
 * un-rotated at their source positions and re-rotated at their target
 * positions) — and, for paged caches, the per-token slot of every block
 * table entry (knlp "Routing", request-flow figure). */
size_t helm_kv_workspace_bytes(const helm_shape_t* shape);
size_t helm_kv_paged_workspace_bytes(const helm_paged_shape_t* shape);

/* Which kernel a helm_kv_transfer call with exactly these arguments would
 * run, without enqueueing anything (so a caller can see the performance
 * class of a call before making it).  Same arguments and the same checks as
 * helm_kv_transfer; on HELM_OK, *path_out is
 *   HELM_PATH_MATRIX    the matrix-core kernel (bf16, head_dim 128,
 *                       1 <= k <= 4, every tensor 16-byte aligned, every
 *                       cache slab and output below 4 GB of addressing);
 *   HELM_PATH_PORTABLE  the portable fp32 vector-ALU kernel (fp32 storage,
 *                       head_dim 64, k > 4 or a misaligned view): the same
 *                       results within tolerance, several times slower.
 * The paged transfer follows the same rule on its pools.  Does not touch
 * the device beyond the arch gate; the workspace fields may be zero. */
#define HELM_PATH_MATRIX 1
#define HELM_PATH_PORTABLE 2
int helm_kv_transfer_path(const void* src_k, const void* src_v,
                          const int32_t* src_pos, const int32_t* tgt_pos,
                          const int32_t* layer_sel,
                          const void* W_k, const float* b_k,
                          const void* W_v, const float* b_v,
                          void* out_k, void* out_v,
                          const helm_shape_t* shape, int* path_out);

/* Registration-time check of a mapper ("Helm Intelligent Routing", section
 * "Requirements": an impossible pair is refused with the specific reason
 * when it is registered).  layer_sel_host: HOST copy [L_t, k].  Checks the
 * shape fields and that every entry lies in [0, L_s).  No device access. */
int helm_mapper_check(const helm_shape_t* shape, const int32_t* layer_sel_host);

/* Host-side check of a paged batch: cu_seqlens starts at 0, is
 * non-decreasing and ends at n_tokens_total; every request fits its table
 * rows; every used block id lies inside its pool; the used target block ids
 * are pairwise distinct (so no two tokens race for a slot).  All pointers
 * are HOST copies.  No device access. */
int helm_paged_check(const helm_paged_shape_t* shape,
                     const int32_t* src_block_table_host,
                     const int32_t* tgt_block_table_host,
                     const int32_t* cu_seqlens_host);

/* Checks that `device` (or the current device when device < 0) exists and
 * is a gfx950 part.  HELM_E_NO_DEVICE / HELM_E_ARCH otherwise (hardware the
 * gate refuses keeps the whole feature off: "Helm Intelligent Routing",
 * section "Safety rails that always apply"). */
int helm_device_check(int device);

/* Pure function behind the arch gate: 1 when a gcnArchName string (e.g.
 * "gfx950:sramecc+:xnack-") names a supported target, else 0. */
int helm_arch_supported(const char* gcn_arch_name);

/* The calling thread's last error text ("" after success): the specific
 * reason for a refusal, with the offending value ("Helm Intelligent
 * Routing", section "Requirements": an impossible pair is refused at
 * registration with the specific reason).  Owned by the library; valid
 * until the thread's next call. */
const char* helm_last_error(void);

/* Static name of a status code ("HELM_OK", ...; "unknown" otherwise), so a
 * caller can log the typed refusal it falls back on ("Helm Intelligent
 * Routing", section "What happens when a transfer cannot be used"). */
const char* helm_status_string(int status);

/* HELM_ABI_VERSION of the built library: a caller that registers mappers
 * against this header can check at load time that the library it found
 * takes the same structures ("Helm Intelligent Routing", section
 * "Requirements": an incompatible pairing is refused up front rather than
 * failing later). */
int helm_abi_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* HELM_KV_H */
