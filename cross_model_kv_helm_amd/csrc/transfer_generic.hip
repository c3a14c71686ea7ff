// transfer_generic.hip — the portable transfer kernel (fp32 vector units).
//
// Serves the fp32 storage dtype and any bf16 shape the matrix-core kernel
// does not take.  One workgroup maps one token tile of one (target layer,
// head, K|V) group:
//   1. gather the group's k selected source layers for the tile's tokens and,
//      for keys, un-rotate them at src_pos (the Qwen3 cache-mapping write-up,
//      section "A linear bridge, strangely enough, suffices": strip the
//      source RoPE; concatenate the selected layers' features); with bf16
//      storage the content key is rounded once to bf16, the operand type of
//      the map;
//   2. y = x W + b in fp32, W in-major as in that section's listing;
//   3. for keys, re-rotate at tgt_pos — always ("Helm Intelligent Routing",
//      section "Why carrying the cache across is the hard part": step 3 is
//      not optional) — and store in the storage dtype (nearest-even).
#include "internal.hpp"

namespace helm {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsBudget = 64 * 1024;

__device__ __forceinline__ float load_as_f32(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ float load_as_f32(const float* p, int64_t i) { return p[i]; }

__device__ __forceinline__ void store_from_f32(uint16_t* p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);   // round to nearest even
}
__device__ __forceinline__ void store_from_f32(float* p, int64_t i, float v) { p[i] = v; }

__device__ __forceinline__ float to_operand(float x, const uint16_t*) { return (float)(__bf16)x; }
__device__ __forceinline__ float to_operand(float x, const float*) { return x; }

template <typename T>
__global__ void __launch_bounds__(kThreads)
transfer_generic_kernel(XferArgs a, int32_t tile) {
  extern __shared__ float xs[];               // [tile][k*D]
  __shared__ int32_t sel[64];
  const int32_t D = a.D, half = D / 2, kD = a.k * D;
  const int32_t grp = blockIdx.y;             // l * H + h
  const int32_t l = grp / a.H, h = grp - l * a.H;
  const bool is_k = blockIdx.z == 0;
  const int64_t n0 = (int64_t)blockIdx.x * tile;

  if (threadIdx.x < a.k) sel[threadIdx.x] = a.layer_sel[(int64_t)l * a.k + threadIdx.x];
  __syncthreads();
  for (int j = 0; j < a.k; ++j)
    if (sel[j] < 0 || sel[j] >= a.L_s) return;   // invalid mapper row: write nothing

  const T* src = (const T*)(is_k ? a.src_k : a.src_v);
  for (int32_t idx = threadIdx.x; idx < tile * kD; idx += kThreads) {
    const int32_t tt = idx / kD, m = idx - tt * kD;
    const int32_t j = m / D, d = m - j * D;
    const int64_t n = n0 + tt;
    float x = 0.f;
    if (n < a.n_tok) {
      const int64_t row = a.src_row ? (int64_t)a.src_row[n] : n;
      if (row >= 0) {
        const int64_t base = (int64_t)sel[j] * a.src_layer + (int64_t)h * a.src_head + row * a.src_tok;
        if (is_k) {
          const int32_t i = d < half ? d : d - half;
          const float2 cs = a.rope_src[rope_src_index(n, i, half)];
          const float lo = load_as_f32(src, base + i), hi = load_as_f32(src, base + i + half);
          // R(-p): (lo, hi) -> (lo c + hi s, hi c - lo s)
          x = d < half ? fmaf(lo, cs.x, hi * cs.y) : fmaf(hi, cs.x, -(lo * cs.y));
          x = to_operand(x, src);
        } else {
          x = load_as_f32(src, base + d);
        }
      }
    }
    xs[idx] = x;
  }
  __syncthreads();

  const T* W = (const T*)(is_k ? a.W_k : a.W_v) + (int64_t)grp * kD * D;
  const float* b = (is_k ? a.b_k : a.b_v) + (int64_t)grp * D;
  T* out = (T*)(is_k ? a.out_k : a.out_v);
  for (int32_t p = threadIdx.x; p < tile * half; p += kThreads) {
    const int32_t tt = p / half, i = p - tt * half;
    const int64_t n = n0 + tt;
    if (n >= a.n_tok) continue;
    const int64_t row = a.dst_row ? (int64_t)a.dst_row[n] : n;
    if (row < 0) continue;
    float y_lo = b[i], y_hi = b[i + half];
    const float* x = xs + tt * kD;
    for (int32_t m = 0; m < kD; ++m) {
      y_lo = fmaf(x[m], load_as_f32(W, (int64_t)m * D + i), y_lo);
      y_hi = fmaf(x[m], load_as_f32(W, (int64_t)m * D + i + half), y_hi);
    }
    float o_lo = y_lo, o_hi = y_hi;
    if (is_k) {  // R(+p'): (lo, hi) -> (lo c - hi s, hi c + lo s)
      const float2 cs = a.rope_tgt[rope_tgt_index(n, i, half)];
      o_lo = fmaf(y_lo, cs.x, -(y_hi * cs.y));
      o_hi = fmaf(y_hi, cs.x, y_lo * cs.y);
    }
    const int64_t base = (int64_t)l * a.dst_layer + (int64_t)h * a.dst_head + row * a.dst_tok;
    store_from_f32(out, base + i, o_lo);
    store_from_f32(out, base + i + half, o_hi);
  }
}

}  // namespace

hipError_t launch_transfer_generic(const XferArgs& a, Dtype dt, hipStream_t stream) {
  if (a.n_tok <= 0) return hipSuccess;
  const int32_t kD = a.k * a.D;
  int32_t tile = kLdsBudget / (kD * 4);
  if (tile > 32) tile = 32;
  if (tile < 1) return hipErrorInvalidValue;
  const int64_t n_tiles = (a.n_tok + tile - 1) / tile;
  if (n_tiles > 0x7fffffff || (int64_t)a.L_t * a.H > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_tiles, (unsigned)(a.L_t * a.H), 2);
  const size_t lds = (size_t)tile * kD * sizeof(float);
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(transfer_generic_kernel<uint16_t>, grid, dim3(kThreads), lds, stream, a, tile);
  else
    hipLaunchKernelGGL(transfer_generic_kernel<float>, grid, dim3(kThreads), lds, stream, a, tile);
  return hipGetLastError();
}

}  // namespace helm
