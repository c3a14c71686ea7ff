// internal.hpp — declarations shared by the library's translation units.
// Not installed; the public interface is include/helm_kv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace helm {

// One transfer, in the form every kernel consumes.  Source rows and target
// rows are addressed through strides so that the contiguous layout
// [L, H, T, D] and the paged layout [L, n_blocks * block_size, H, D] share
// the kernels:
//   source element (s, h, n, d) = src + s*src_layer + h*src_head + row*src_tok + d
// with row = n (contiguous) or row = src_row[n] (paged, -1 = skip token).
struct XferArgs {
  const void* src_k;
  const void* src_v;
  const int32_t* layer_sel;   // [L_t, k]
  const void* W_k;            // [L_t, H, k*D, D]
  const float* b_k;           // [L_t, H, D]
  const void* W_v;
  const float* b_v;
  void* out_k;
  void* out_v;
  const float2* rope_src;     // (cos, sin) at src_pos, theta_src, in rope_src_index layout
  const float2* rope_tgt;     // (cos, sin) at tgt_pos, theta_tgt, in rope_tgt_index layout
  const int32_t* src_row;     // [n_tok] or nullptr (identity)
  const int32_t* dst_row;     // [n_tok] or nullptr (identity)
  int64_t n_tok;
  int64_t src_rows, dst_rows;   // rows addressable per (layer, head): T, or pool slots
  int32_t L_s, L_t, H, D, k;
  int64_t src_layer, src_head, src_tok;   // element strides
  int64_t dst_layer, dst_head, dst_tok;
};

enum class Dtype : int { BF16 = 0, F32 = 1 };

// Layouts of the (cos, sin) tables written by K1, blocked by 16-token tiles
// (the matrix-core kernel's token tile) and different for the two sides, so
// that each side's readers make contiguous 16-byte accesses.  half = D/2 (a
// multiple of 8); within the block of tokens [16b, 16b+16), with tt = t%16,
// pair i of token t lives at float2 index b*16*half + ...:
//   source table (read by the gather/un-rotation: one 16-byte piece of pairs
//   (8c + 2e, 8c + 2e + 1) per lane):  e*4*half + tt*(half/4) + (i/8)*2 + i%2,
//   with e = (i%8)/2, i.e. [e][tt][i/8][2 pairs];
//   target table (read by the epilogue: pairs 4g .. 4g+3 of a token as two
//   16-byte halves):  (i/4)*64 + ((i%4)/2)*32 + tt*2 + i%2,
//   i.e. [i/4][(i%4)/2][tt][2 pairs].
constexpr int kRopeBlock = 16;
__host__ __device__ inline int64_t rope_src_index(int64_t t, int32_t i, int32_t half) {
  const int64_t b = t / kRopeBlock;
  const int32_t tt = (int32_t)(t - b * kRopeBlock);
  return b * kRopeBlock * half + (int64_t)((i & 7) >> 1) * (4 * half) + (int64_t)tt * (half / 4) + (i >> 3) * 2 +
         (i & 1);
}
__host__ __device__ inline int64_t rope_tgt_index(int64_t t, int32_t i, int32_t half) {
  const int64_t b = t / kRopeBlock;
  const int32_t tt = (int32_t)(t - b * kRopeBlock);
  return b * kRopeBlock * half + (int64_t)(i >> 2) * 64 + ((i & 3) >> 1) * 32 + tt * 2 + (i & 1);
}
inline int64_t rope_table_entries(int64_t n_tok, int32_t half) {
  return (n_tok + kRopeBlock - 1) / kRopeBlock * kRopeBlock * half;
}

// K1: cos/sin tables of the RoPE angles for src_pos and tgt_pos.
hipError_t launch_rope_tables(const int32_t* src_pos, const int32_t* tgt_pos, int64_t n_tok,
                              int32_t D, double theta_src, double theta_tgt,
                              float2* rope_src, float2* rope_tgt, hipStream_t stream);

// Paged prologue: per packed token, the physical source and target slot
// (block * block_size + offset), or -1 when a table entry is out of range.
hipError_t launch_paged_rows(const int32_t* cu_seqlens, int32_t n_requests,
                             const int32_t* src_bt, int32_t max_blocks_src, int32_t n_src_blocks,
                             const int32_t* tgt_bt, int32_t max_blocks_tgt, int32_t n_tgt_blocks,
                             int32_t block_size, int64_t n_tok,
                             int32_t* src_row, int32_t* dst_row, hipStream_t stream);

// Portable transfer kernel: fp32 vector arithmetic, any supported D/k/dtype.
hipError_t launch_transfer_generic(const XferArgs& a, Dtype dt, hipStream_t stream);

// KV-cosine diagnostic: out[kv * n_slabs + s] = cosine of slab s of the
// mapped and the reference cache (kv = 0 keys, 1 values), slabs of
// slab_elems values each.
hipError_t launch_kv_cosine(const void* k_a, const void* v_a, const void* k_b, const void* v_b, int64_t n_slabs,
                            int64_t slab_elems, Dtype dt, float* out, hipStream_t stream);

// Wide-input map (bf16, head_dim 128): x = the K (un-rotated) and V features
// of all heads of the k selected source layers, IN = k*2*H*D; one (IN, D) map
// per target head and K|V.  U, WT_k, WT_v are workspace: the un-rotated keys
// [L_s, H, T, D] and the transposed maps [L_t, H, D, IN].
struct WideXfer {
  const void* src_k;
  const void* src_v;
  const int32_t* layer_sel;   // [L_t, k]
  const void* W_k;            // [L_t, H, IN, D]
  const float* b_k;           // [L_t, H, D]
  const void* W_v;
  const float* b_v;
  void* out_k;                // [L_t, H, T, D]
  void* out_v;
  const float2* rope_src;     // K1 tables (rope_src_index / rope_tgt_index layouts)
  const float2* rope_tgt;
  uint16_t* U;
  uint16_t* WT_k;
  uint16_t* WT_v;
  int32_t L_s, L_t, H, D, k, T;
};
int64_t wide_in_features(int32_t k, int32_t H, int32_t D);
bool wide_supports(const WideXfer& x);
// prep: the un-rotated keys and the transposed maps into the workspace
// (reads rope_src); product: the map itself, reading them.
hipError_t launch_wide(const WideXfer& x, bool prep, bool product, hipStream_t stream);

// Ridge fit of G maps (bf16 observations, D = 128 targets, IN a multiple of
// 128 up to 1024): gram/cross/sums/shift/M are workspace, W [G, IN, D] and
// b [G, D] the fp32 results.
struct RidgeFit {
  const void* X;     // [G, N, IN] bf16
  const void* Y;     // [G, N, D] bf16
  float* gram;       // [G, IN, IN]
  float* cross;      // [G, IN, D]
  float* sums;       // [G, IN + D]
  float* shift;      // [G, IN + D]
  double* M;         // [G, IN, IN + D]
  float* W;
  float* b;
  int64_t G, N;
  int32_t IN, D;
  double lambda;
};
int64_t ridge_tiles_per_group(int32_t IN);
bool ridge_supports(const RidgeFit& f);
// gram: the products and sums into the workspace; solve: the fit from them.
hipError_t launch_ridge(const RidgeFit& f, bool gram, bool solve, hipStream_t stream);

// Matrix-core transfer kernel for bf16 storage.  Returns hipErrorNotSupported
// (and enqueues nothing) when the shape is outside what it handles.
hipError_t launch_transfer_mfma(const XferArgs& a, hipStream_t stream);
bool mfma_supports(const XferArgs& a);

}  // namespace helm
