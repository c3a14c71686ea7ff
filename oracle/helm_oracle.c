/*
 * helm_oracle.c — the fp64 CPU oracle of the cross-model KV-cache transfer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the transfer computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * source, header, table or helper with the HIP library under
 * cross_model_kv_helm_amd/, and the library never calls it.
 *
 * What it follows (page titles and sections; no line numbers):
 *   - "Helm Intelligent Routing", section "Why carrying the cache across is the
 *     hard part": the pilot's keys are un-rotated back into content space, a
 *     per-layer, per-head linear map fitted offline converts them, and the
 *     result is re-rotated at the position it will occupy in the target;
 *     the re-rotation is never skipped.
 *   - "Moving the KV cache between Qwen3 models instead of re-prefilling"
 *     (Russian write-up), section "A linear bridge, strangely enough,
 *     suffices": select useful source layers and concatenate their features;
 *     fit keys and values separately per target layer and head; the map is
 *     x @ w + b with w of shape (in, out); strip the source RoPE, map the
 *     position-free content, apply the target RoPE (the diagram there).
 *   - "Helm Intelligent Routing", section "Requirements": both models share
 *     the KV-head count and the per-head dimension; layer counts may differ.
 *   - knlp "Routing" page, request-flow figure: block tables name the pages of
 *     a request in a paged cache; writes go only to the selected blocks.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - RoPE is the rotate-half form: dimension i pairs with i + D/2, angular
 *     frequency w_i = theta^(-2i/D), and R(p) turns each pair by p*w_i
 *     counter-clockwise: (a, b) -> (a cos - b sin, b cos + a sin).
 *   - The concatenation order of the selected source layers is the order of
 *     the layer_sel row as given.
 *   - W is stored in-major [k*D][D]; y[n] = b[n] + sum_m x[m] W[m][n].
 *   - The bias is added in content space, before the forward rotation.
 *   - Values carry no position and are never rotated.
 *   - "quantize_content" mode rounds the un-rotated key to the storage dtype
 *     (round to nearest, ties to even) before the map: the map is a bf16
 *     contraction, so its key operand is bf16 by definition.  This is the
 *     only rounding point; everything else is fp64 and the result is fp64.
 *
 * Angles are formed in fp64 (p * w_i with p an exact integer) and passed to
 * libm cos/sin, which reduce the argument themselves.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1

typedef struct {
  int32_t n_src_layers;   /* L_s */
  int32_t n_tgt_layers;   /* L_t */
  int32_t n_kv_heads;     /* H, the same on both sides */
  int32_t head_dim;       /* D, the same on both sides, even */
  int32_t k;              /* selected source layers per target layer */
  int32_t dtype;          /* ORACLE_BF16 (uint16 storage) or ORACLE_F32 */
  int32_t quantize_content; /* 1: round the un-rotated key to dtype first */
  int32_t n_threads;      /* <= 0: OpenMP default */
  int64_t n_tokens;       /* T (contiguous layout) */
  double theta_src;
  double theta_tgt;
} oracle_problem;

/* ------------------------------------------------------------------ */
/* Storage formats                                                     */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper 16 bits of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == ORACLE_BF16) return bf16_to_double(((const uint16_t*)base)[idx]);
  return (double)((const float*)base)[idx];
}

/* Round an fp64 value once to the nearest bf16 value (8 significant bits,
 * binary32 exponent range), ties to even.  Result returned as fp64. */
double oracle_round_bf16(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);                       /* |x| in [2^(e-1), 2^e) */
  if (e - 1 < -126) e = -125;         /* subnormal bf16: fixed quantum 2^-133 */
  double q = ldexp(1.0, e - 8);       /* spacing of bf16 values in that binade */
  double r = nearbyint(x / q) * q;    /* x / q is exact: q is a power of two */
  const double max_bf16 = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > max_bf16) r = copysign(INFINITY, x);
  return r;
}

/* Round an fp64 value once to the nearest binary32 value, ties to even. */
double oracle_round_f32(double x) { return (double)(float)x; }

static double round_to_dtype(double x, int32_t dtype) {
  return dtype == ORACLE_BF16 ? oracle_round_bf16(x) : oracle_round_f32(x);
}

/* ------------------------------------------------------------------ */
/* RoPE, rotate-half form                                              */
/* ------------------------------------------------------------------ */

/* Angular frequency of pair i for head dimension D and base theta. */
double oracle_rope_freq(int32_t i, int32_t D, double theta) {
  return pow(theta, -2.0 * (double)i / (double)D);
}

/* out = R(p; theta) * in, for one D-vector (in and out may alias). */
void oracle_rope(const double* in, double* out, int32_t D, double p, double theta) {
  const int32_t half = D / 2;
  for (int32_t i = 0; i < half; ++i) {
    double a = p * oracle_rope_freq(i, D, theta);
    double c = cos(a), s = sin(a);
    double lo = in[i], hi = in[i + half];
    out[i] = lo * c - hi * s;
    out[i + half] = hi * c + lo * s;
  }
}

/* ------------------------------------------------------------------ */
/* One output row of the transfer                                      */
/* ------------------------------------------------------------------ */

/* Everything one row needs, resolved by the caller (contiguous or paged). */
typedef struct {
  const void* src_k;   /* base of the source K cache / pool */
  const void* src_v;
  const int64_t* src_row_off; /* [k]: element offset of the D-vector in src */
  int64_t src_pos;
  int64_t tgt_pos;
  const void* W_k;     /* this (target layer, head)'s [k*D][D] block */
  const void* W_v;
  const float* b_k;    /* this (target layer, head)'s [D] bias */
  const float* b_v;
} row_inputs;

/* Computes out_k[D], out_v[D] for one (target layer, head, token).
 * scratch must hold 3*k*D + 2*D doubles. */
static void transfer_one_row(const oracle_problem* pb, const row_inputs* in,
                             double* out_k, double* out_v, double* scratch) {
  const int32_t D = pb->head_dim, k = pb->k, KD = k * D;
  double* xk = scratch;          /* [k*D] un-rotated keys, concatenated */
  double* xv = xk + KD;          /* [k*D] values, concatenated */
  double* u = xv + KD;           /* [k*D] staging */
  double* yk = u + KD;           /* [D] */
  double* yv = yk + D;           /* [D] */

  /* Step 1 + gather: for each selected layer, un-rotate the stored key at
   * its source position, R(-p) = R(p)^-1, and place it in row block j. */
  for (int32_t j = 0; j < k; ++j) {
    for (int32_t d = 0; d < D; ++d) {
      u[j * D + d] = load_elem(in->src_k, pb->dtype, in->src_row_off[j] + d);
      xv[j * D + d] = load_elem(in->src_v, pb->dtype, in->src_row_off[j] + d);
    }
    oracle_rope(u + j * D, xk + j * D, D, -(double)in->src_pos, pb->theta_src);
  }
  if (pb->quantize_content)
    for (int32_t m = 0; m < KD; ++m) xk[m] = round_to_dtype(xk[m], pb->dtype);

  /* Step 2: y = x @ W + b, W in-major. */
  for (int32_t n = 0; n < D; ++n) {
    yk[n] = (double)in->b_k[n];
    yv[n] = (double)in->b_v[n];
  }
  for (int32_t m = 0; m < KD; ++m) {
    const double a = xk[m], v = xv[m];
    for (int32_t n = 0; n < D; ++n) {
      yk[n] += a * load_elem(in->W_k, pb->dtype, (int64_t)m * D + n);
      yv[n] += v * load_elem(in->W_v, pb->dtype, (int64_t)m * D + n);
    }
  }

  /* Step 3: re-rotate the mapped key at its target position; always. */
  oracle_rope(yk, out_k, D, (double)in->tgt_pos, pb->theta_tgt);
  for (int32_t n = 0; n < D; ++n) out_v[n] = yv[n];
}

static int check_problem(const oracle_problem* pb) {
  if (!pb) return 1;
  if (pb->n_src_layers <= 0 || pb->n_tgt_layers <= 0 || pb->n_kv_heads <= 0) return 1;
  if (pb->head_dim <= 0 || (pb->head_dim & 1)) return 1;
  if (pb->k <= 0) return 1;
  if (pb->dtype != ORACLE_BF16 && pb->dtype != ORACLE_F32) return 1;
  return 0;
}

static void set_threads(const oracle_problem* pb) {
#ifdef _OPENMP
  if (pb->n_threads > 0) omp_set_num_threads(pb->n_threads);
#else
  (void)pb;
#endif
}

/* ------------------------------------------------------------------ */
/* Contiguous layout: caches [L, H, T, D], W [L_t, H, k*D, D],          */
/* bias [L_t, H, D], layer_sel [L_t, k], positions [T].                 */
/* ------------------------------------------------------------------ */

/* rows: flat indices (l*H + h)*T + t; NULL means every row in order.
 * out_k / out_v: [n_rows, D] fp64.  Returns 0, or 1 on a bad argument
 * (including a layer_sel entry outside [0, L_s)). */
int oracle_transfer_rows(const oracle_problem* pb,
                         const void* src_k, const void* src_v,
                         const int32_t* src_pos, const int32_t* tgt_pos,
                         const int32_t* layer_sel,
                         const void* W_k, const float* b_k,
                         const void* W_v, const float* b_v,
                         int64_t n_rows, const int64_t* rows,
                         double* out_k, double* out_v) {
  if (check_problem(pb) || pb->n_tokens <= 0) return 1;
  const int64_t T = pb->n_tokens, H = pb->n_kv_heads, D = pb->head_dim;
  const int32_t k = pb->k;
  const int64_t total = (int64_t)pb->n_tgt_layers * H * T;
  if (!rows) n_rows = total;
  for (int64_t j = 0; j < (int64_t)pb->n_tgt_layers * k; ++j)
    if (layer_sel[j] < 0 || layer_sel[j] >= pb->n_src_layers) return 1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return 1;

  set_threads(pb);
  int bad = 0;
#pragma omp parallel
  {
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(3 * k * D + 2 * D));
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
    if (!scratch || !off) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t t = flat % T;
        const int64_t h = (flat / T) % H;
        const int64_t l = flat / (T * H);
        for (int32_t j = 0; j < k; ++j) {
          const int64_t s = layer_sel[l * k + j];
          off[j] = ((s * H + h) * T + t) * D;
        }
        const int64_t grp = l * H + h;
        const size_t wbytes = pb->dtype == ORACLE_BF16 ? 2 : 4;
        row_inputs in = {
            src_k, src_v, off, src_pos[t], tgt_pos[t],
            (const char*)W_k + (size_t)grp * (size_t)(k * D * D) * wbytes,
            (const char*)W_v + (size_t)grp * (size_t)(k * D * D) * wbytes,
            b_k + grp * D, b_v + grp * D};
        transfer_one_row(pb, &in, out_k + r * D, out_v + r * D, scratch);
      }
    }
    free(scratch);
    free(off);
  }
  return bad;
}

/* ------------------------------------------------------------------ */
/* Wide-input map                                                       */
/* ------------------------------------------------------------------ */

/* The Qwen3 cache-mapping write-up, section "A linear bridge, strangely
 * enough, suffices": the full mapper's x concatenates the KV features of all
 * selected source layers, and every target head has its own fits (one for
 * keys, one for values); its parameter count (about 1.07 B for 14B -> 32B)
 * is 64 layers x 8 heads x {K, V} x (IN*128 + 128) with IN = 8192 =
 * k x {K, V} x H x D.  Readings (the text gives no order):
 *   x[((j*2 + kv)*H + g)*D + d] = kv == 0 ? (R(-src_pos[t]) src_k[sel_j, g, t, :])[d]
 *                                         : src_v[sel_j, g, t, d]
 * with sel_j = layer_sel[l, j] in row order, keys before values, source head
 * g, dimension d; keys are un-rotated (and, in quantize_content mode, rounded
 * once to the storage dtype) exactly as in the per-head map.  Then
 *   out_k[l, h, t, :] = R(+tgt_pos[t]) (x @ W_k[l, h] + b_k[l, h])
 *   out_v[l, h, t, :] = x @ W_v[l, h] + b_v[l, h]
 * with W_* [L_t, H, IN, D] in-major and b_* [L_t, H, D].
 * rows: flat indices (l*H + h)*T + t (NULL = all, in order); out_k / out_v:
 * [n_rows, D] fp64.  Returns 0, or 1 on a bad argument. */
int oracle_transfer_wide_rows(const oracle_problem* pb,
                              const void* src_k, const void* src_v,
                              const int32_t* src_pos, const int32_t* tgt_pos,
                              const int32_t* layer_sel,
                              const void* W_k, const float* b_k,
                              const void* W_v, const float* b_v,
                              int64_t n_rows, const int64_t* rows,
                              double* out_k, double* out_v) {
  if (check_problem(pb) || pb->n_tokens <= 0) return 1;
  const int64_t T = pb->n_tokens, H = pb->n_kv_heads, D = pb->head_dim;
  const int32_t k = pb->k;
  const int64_t IN = (int64_t)k * 2 * H * D;
  const int64_t total = (int64_t)pb->n_tgt_layers * H * T;
  if (!rows) n_rows = total;
  for (int64_t j = 0; j < (int64_t)pb->n_tgt_layers * k; ++j)
    if (layer_sel[j] < 0 || layer_sel[j] >= pb->n_src_layers) return 1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return 1;
  const size_t wbytes = pb->dtype == ORACLE_BF16 ? 2 : 4;

  set_threads(pb);
  int bad = 0;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(IN + 3 * D));
    if (!x) {
#pragma omp atomic write
      bad = 1;
    } else {
      double* u = x + IN;     /* [D] staging */
      double* yk = u + D;     /* [D] */
      double* yv = yk + D;    /* [D] */
#pragma omp for schedule(static)
      for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t t = flat % T;
        const int64_t h = (flat / T) % H;
        const int64_t l = flat / (T * H);
        /* gather: layer j, then keys (un-rotated) before values, then head g */
        for (int32_t j = 0; j < k; ++j) {
          const int64_t s = layer_sel[l * k + j];
          for (int64_t g = 0; g < H; ++g) {
            const int64_t src = ((s * H + g) * T + t) * D;
            double* xk = x + ((int64_t)(j * 2 + 0) * H + g) * D;
            double* xv = x + ((int64_t)(j * 2 + 1) * H + g) * D;
            for (int64_t d = 0; d < D; ++d) {
              u[d] = load_elem(src_k, pb->dtype, src + d);
              xv[d] = load_elem(src_v, pb->dtype, src + d);
            }
            oracle_rope(u, xk, (int32_t)D, -(double)src_pos[t], pb->theta_src);
            if (pb->quantize_content)
              for (int64_t d = 0; d < D; ++d) xk[d] = round_to_dtype(xk[d], pb->dtype);
          }
        }
        const int64_t grp = l * H + h;
        const char* wk = (const char*)W_k + (size_t)grp * (size_t)(IN * D) * wbytes;
        const char* wv = (const char*)W_v + (size_t)grp * (size_t)(IN * D) * wbytes;
        for (int64_t n = 0; n < D; ++n) {
          yk[n] = (double)b_k[grp * D + n];
          yv[n] = (double)b_v[grp * D + n];
        }
        for (int64_t m = 0; m < IN; ++m) {
          const double a = x[m];
          for (int64_t n = 0; n < D; ++n) {
            yk[n] += a * load_elem(wk, pb->dtype, m * D + n);
            yv[n] += a * load_elem(wv, pb->dtype, m * D + n);
          }
        }
        oracle_rope(yk, out_k + r * D, (int32_t)D, (double)tgt_pos[t], pb->theta_tgt);
        for (int64_t n = 0; n < D; ++n) out_v[r * D + n] = yv[n];
      }
    }
    free(x);
  }
  return bad;
}

/* ------------------------------------------------------------------ */
/* Paged layout: pools [L, n_blocks, block_size, H, D]; block tables    */
/* [R, max_blocks]; cu_seqlens [R+1]; positions [N] over packed tokens. */
/* Token t of request r sits in slot t % block_size of logical page     */
/* t / block_size, whose physical block id is bt[r][t / block_size].    */
/* ------------------------------------------------------------------ */

typedef struct {
  int32_t block_size;
  int32_t n_requests;
  int32_t max_blocks_src, max_blocks_tgt;  /* row strides of the tables */
  int32_t n_src_blocks, n_tgt_blocks;      /* pool sizes (blocks) */
} oracle_paged;

/* Finds the request that owns packed token n: cu[r] <= n < cu[r+1]. */
static int32_t owner_request(const int32_t* cu, int32_t R, int64_t n) {
  int32_t lo = 0, hi = R;  /* invariant: cu[lo] <= n < cu[hi] */
  while (hi - lo > 1) {
    int32_t mid = lo + (hi - lo) / 2;
    if (cu[mid] <= n) lo = mid; else hi = mid;
  }
  return lo;
}

/* rows: flat indices (l*H + h)*N + n over packed tokens n < N = cu[R].
 * out_k / out_v: [n_rows, D] fp64.  dst_off (optional): [n_rows] element
 * offset of the row's destination in the target pool [L_t, n_tgt_blocks,
 * block_size, H, D].  Returns 0, or 1 on a bad argument. */
int oracle_transfer_paged_rows(const oracle_problem* pb, const oracle_paged* pg,
                               const void* src_k_pool, const void* src_v_pool,
                               const int32_t* src_bt, const int32_t* tgt_bt,
                               const int32_t* cu_seqlens,
                               const int32_t* src_pos, const int32_t* tgt_pos,
                               const int32_t* layer_sel,
                               const void* W_k, const float* b_k,
                               const void* W_v, const float* b_v,
                               int64_t n_rows, const int64_t* rows,
                               double* out_k, double* out_v, int64_t* dst_off) {
  if (check_problem(pb) || !pg || pg->block_size <= 0 || pg->n_requests <= 0) return 1;
  const int32_t R = pg->n_requests, B = pg->block_size;
  const int64_t H = pb->n_kv_heads, D = pb->head_dim;
  const int32_t k = pb->k;
  if (cu_seqlens[0] != 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    const int64_t len = (int64_t)cu_seqlens[r + 1] - cu_seqlens[r];
    if (len < 0) return 1;
    if ((len + B - 1) / B > pg->max_blocks_src || (len + B - 1) / B > pg->max_blocks_tgt) return 1;
  }
  const int64_t N = cu_seqlens[R];
  const int64_t total = (int64_t)pb->n_tgt_layers * H * N;
  if (!rows) n_rows = total;
  for (int64_t j = 0; j < (int64_t)pb->n_tgt_layers * k; ++j)
    if (layer_sel[j] < 0 || layer_sel[j] >= pb->n_src_layers) return 1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return 1;

  set_threads(pb);
  int bad = 0;
#pragma omp parallel
  {
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(3 * k * D + 2 * D));
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
    if (!scratch || !off) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t n = flat % N;
        const int64_t h = (flat / N) % H;
        const int64_t l = flat / (N * H);
        const int32_t req = owner_request(cu_seqlens, R, n);
        const int64_t t = n - cu_seqlens[req];
        const int64_t page = t / B, slot = t % B;
        const int64_t sblk = src_bt[(int64_t)req * pg->max_blocks_src + page];
        const int64_t tblk = tgt_bt[(int64_t)req * pg->max_blocks_tgt + page];
        if (sblk < 0 || sblk >= pg->n_src_blocks || tblk < 0 || tblk >= pg->n_tgt_blocks) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        for (int32_t j = 0; j < k; ++j) {
          const int64_t s = layer_sel[l * k + j];
          off[j] = (((s * pg->n_src_blocks + sblk) * B + slot) * H + h) * D;
        }
        const int64_t grp = l * H + h;
        const size_t wbytes = pb->dtype == ORACLE_BF16 ? 2 : 4;
        row_inputs in = {
            src_k_pool, src_v_pool, off, src_pos[n], tgt_pos[n],
            (const char*)W_k + (size_t)grp * (size_t)(k * D * D) * wbytes,
            (const char*)W_v + (size_t)grp * (size_t)(k * D * D) * wbytes,
            b_k + grp * D, b_v + grp * D};
        transfer_one_row(pb, &in, out_k + r * D, out_v + r * D, scratch);
        if (dst_off) dst_off[r] = (((l * pg->n_tgt_blocks + tblk) * B + slot) * H + h) * D;
      }
    }
    free(scratch);
    free(off);
  }
  return bad;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Input preparation for tests: position-encode content keys           */
/* ------------------------------------------------------------------ */

/* out[l, h, t, :] = round_dtype(R(pos[t]; theta) in[l, h, t, :]) for a cache
 * [n_layers, H, T, D] stored in dtype (same storage for in and out; they may
 * alias).  This is how a model leaves keys in its cache: rotated at the
 * position each token was produced at.  The cos/sin of a token's angles are
 * evaluated once per token and reused for its n_layers*H rows.
 * Returns 0, or 1 on a bad argument. */
int oracle_encode_keys(const void* in, void* out, int32_t dtype,
                       int64_t n_layers, int64_t H, int64_t T, int32_t D,
                       const int32_t* pos, double theta, int32_t n_threads) {
  if (!in || !out || !pos || n_layers <= 0 || H <= 0 || T <= 0 || D <= 0 || (D & 1)) return 1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return 1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  const int32_t half = D / 2;
  int bad = 0;
#pragma omp parallel
  {
    double* cs = (double*)malloc(sizeof(double) * (size_t)(2 * half));
    if (!cs) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < half; ++i) {
          const double a = (double)pos[t] * oracle_rope_freq(i, D, theta);
          cs[2 * i] = cos(a);
          cs[2 * i + 1] = sin(a);
        }
        for (int64_t lh = 0; lh < n_layers * H; ++lh) {
          const int64_t r = lh * T + t;
          for (int32_t i = 0; i < half; ++i) {
            const double lo = load_elem(in, dtype, r * D + i);
            const double hi = load_elem(in, dtype, r * D + i + half);
            const double o[2] = {lo * cs[2 * i] - hi * cs[2 * i + 1], hi * cs[2 * i] + lo * cs[2 * i + 1]};
            const int64_t idx[2] = {r * D + i, r * D + i + half};
            for (int q = 0; q < 2; ++q) {
              const double v = round_to_dtype(o[q], dtype);
              if (dtype == ORACLE_BF16) {
                float f = (float)v;  /* exact: v is a bf16 value */
                uint32_t u;
                memcpy(&u, &f, sizeof u);
                ((uint16_t*)out)[idx[q]] = (uint16_t)(u >> 16);
              } else {
                ((float*)out)[idx[q]] = (float)v;
              }
            }
          }
        }
      }
    }
    free(cs);
  }
  return bad;
}

/* ------------------------------------------------------------------ */
/* KV-cosine diagnostic                                                 */
/* ------------------------------------------------------------------ */

/* "Helm Intelligent Routing", the retention / KL / KV-cosine table: the KV
 * cosine measures how close a mapped cache is to the target model's own.
 * Reading (the page gives no formula): for each slab s (one K or V cache of
 * one target layer and head, n_elems = T*D values), the cosine between the
 * two slabs taken as flat vectors,
 *   out[s] = sum(a*b) / (sqrt(sum(a*a)) * sqrt(sum(b*b))),
 * in fp64; a slab of zeros gives 0/0 = NaN.  a and b are n_slabs * n_elems
 * values of dtype, slab-major.  Returns 0, or 1 on a bad argument. */
int oracle_kv_cosine(const void* a, const void* b, int32_t dtype, int64_t n_slabs, int64_t n_elems,
                     double* out, int32_t n_threads) {
  if (!a || !b || !out || n_slabs < 0 || n_elems < 0) return 1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return 1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < n_slabs; ++s) {
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int64_t e = 0; e < n_elems; ++e) {
      const double x = load_elem(a, dtype, s * n_elems + e);
      const double y = load_elem(b, dtype, s * n_elems + e);
      ab += x * y;
      aa += x * x;
      bb += y * y;
    }
    out[s] = ab / (sqrt(aa) * sqrt(bb));
  }
  return 0;
}
