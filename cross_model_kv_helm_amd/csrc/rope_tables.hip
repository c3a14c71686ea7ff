// rope_tables.hip — per-token prologue kernels.
//
// K1 writes the cos/sin of every RoPE angle the transfer needs, once per
// token (in the tile-blocked layouts rope_src_index / rope_tgt_index), so the
// transfer kernels never evaluate trigonometry: the angle of
// pair i at position p is p * theta^(-2i/D) (rotate-half RoPE), formed in
// fp64 because at p ~ 1.3e5 an fp32 product alone would be off by ~1e-2 rad;
// cos and sin are evaluated in fp64 and rounded once to fp32.  The pages use
// the rotation without spelling it out ("Helm Intelligent Routing", section
// "Why carrying the cache across is the hard part": keys carry their position
// folded in as a rotation; the Qwen3 cache-mapping write-up, section "A
// linear bridge, strangely enough, suffices": strip the source RoPE, apply
// the target RoPE).
//
// The paged prologue resolves each packed token to its physical source and
// target slot through the block tables (knlp "Routing" page, request-flow
// figure: block tables map a request's logical pages to physical blocks).
#include "internal.hpp"

namespace helm {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
rope_tables_kernel(const int32_t* __restrict__ src_pos, const int32_t* __restrict__ tgt_pos,
                   int64_t n_tok, int32_t half, double theta_src, double theta_tgt,
                   float2* __restrict__ rope_src, float2* __restrict__ rope_tgt) {
  const int64_t total = n_tok * half;
  const double inv_d = -1.0 / (double)half;   // -2i/D = -i/half
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // A thread's pair index stays fixed across its grid-stride steps when the
  // stride is a multiple of half (D = 64, 128, ...): its two frequencies
  // are then evaluated once; otherwise again for every element.
  const bool fixed_i = half > 0 && stride % half == 0;
  int32_t i_w = -1;
  double w_s = 0.0, w_t = 0.0;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const int64_t t = e / half;
    const int32_t i = (int32_t)(e - t * half);
    if (!fixed_i || i != i_w) {
      const double ex = inv_d * (double)i;
      w_s = pow(theta_src, ex);
      w_t = pow(theta_tgt, ex);
      i_w = i;
    }
    double s, c;
    sincos((double)src_pos[t] * w_s, &s, &c);
    rope_src[rope_src_index(t, i, half)] = make_float2((float)c, (float)s);
    sincos((double)tgt_pos[t] * w_t, &s, &c);
    rope_tgt[rope_tgt_index(t, i, half)] = make_float2((float)c, (float)s);
  }
}

__global__ void __launch_bounds__(kThreads)
paged_rows_kernel(const int32_t* __restrict__ cu, int32_t R,
                  const int32_t* __restrict__ src_bt, int32_t max_src, int32_t n_src_blocks,
                  const int32_t* __restrict__ tgt_bt, int32_t max_tgt, int32_t n_tgt_blocks,
                  int32_t bs, int64_t n_tok, int32_t* __restrict__ src_row,
                  int32_t* __restrict__ dst_row) {
  for (int64_t n = (int64_t)blockIdx.x * kThreads + threadIdx.x; n < n_tok;
       n += (int64_t)gridDim.x * kThreads) {
    // owner request: the last r with cu[r] <= n (bounded search)
    int32_t lo = 0, hi = R;
    while (hi - lo > 1) {
      const int32_t mid = lo + (hi - lo) / 2;
      if ((int64_t)cu[mid] <= n) lo = mid; else hi = mid;
    }
    const int64_t t = n - cu[lo];
    int32_t sr = -1, dr = -1;
    if (t >= 0 && n < (int64_t)cu[lo + 1]) {
      const int64_t page = t / bs, off = t - page * bs;
      if (page < max_src) {
        const int32_t b = src_bt[(int64_t)lo * max_src + page];
        if (b >= 0 && b < n_src_blocks) sr = (int32_t)((int64_t)b * bs + off);
      }
      if (page < max_tgt) {
        const int32_t b = tgt_bt[(int64_t)lo * max_tgt + page];
        if (b >= 0 && b < n_tgt_blocks) dr = (int32_t)((int64_t)b * bs + off);
      }
    }
    // a token is mapped only when both of its slots are valid
    src_row[n] = (sr >= 0 && dr >= 0) ? sr : -1;
    dst_row[n] = (sr >= 0 && dr >= 0) ? dr : -1;
  }
}

int grid_for(int64_t work) {
  const int64_t blocks = (work + kThreads - 1) / kThreads;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_rope_tables(const int32_t* src_pos, const int32_t* tgt_pos, int64_t n_tok,
                              int32_t D, double theta_src, double theta_tgt,
                              float2* rope_src, float2* rope_tgt, hipStream_t stream) {
  if (n_tok <= 0) return hipSuccess;
  const int32_t half = D / 2;
  // at most 2,048 workgroups (8 per CU): each thread then takes several
  // tokens of one pair and evaluates that pair's frequencies once
  const int grid = grid_for(n_tok * half) < 2048 ? grid_for(n_tok * half) : 2048;
  hipLaunchKernelGGL(rope_tables_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     src_pos, tgt_pos, n_tok, half, theta_src, theta_tgt, rope_src, rope_tgt);
  return hipGetLastError();
}

hipError_t launch_paged_rows(const int32_t* cu_seqlens, int32_t n_requests,
                             const int32_t* src_bt, int32_t max_blocks_src, int32_t n_src_blocks,
                             const int32_t* tgt_bt, int32_t max_blocks_tgt, int32_t n_tgt_blocks,
                             int32_t block_size, int64_t n_tok,
                             int32_t* src_row, int32_t* dst_row, hipStream_t stream) {
  if (n_tok <= 0) return hipSuccess;
  hipLaunchKernelGGL(paged_rows_kernel, dim3(grid_for(n_tok)), dim3(kThreads), 0, stream,
                     cu_seqlens, n_requests, src_bt, max_blocks_src, n_src_blocks, tgt_bt,
                     max_blocks_tgt, n_tgt_blocks, block_size, n_tok, src_row, dst_row);
  return hipGetLastError();
}

}  // namespace helm
