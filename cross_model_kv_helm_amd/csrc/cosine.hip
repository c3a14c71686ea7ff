// cosine.hip — the KV-cosine diagnostic: how close a mapped cache is to the
// target model's own ("Helm Intelligent Routing", the retention / KL /
// KV-cosine table).  For every slab (the K or V cache of one target layer
// and head, T*D values) the cosine of the two slabs as flat vectors:
//   cos = sum(a*b) / (sqrt(sum(a*a)) * sqrt(sum(b*b)))   (0/0 = NaN).
//
// Design for MI355X: a streaming reduction, bound by HBM (both caches are
// read once, nothing but one float per slab is written).  One 256-thread
// workgroup per slab; each thread streams 16-byte pieces of both slabs
// through buffer descriptors (a piece past the slab reads zeros, so the loop
// needs no tail), four pieces of each in flight.  The three sums of a
// piece are formed in fp32 (at most 8 products) and added into fp64
// accumulators, so a 4M-element slab keeps ~1e-15 relative error in its
// sums; the block reduction and the division are fp64.
#include "internal.hpp"

namespace helm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr uint32_t kMaxSlabBytes = 0xfff00000u;   // one buffer descriptor per slab; base + step cannot wrap

__device__ __forceinline__ rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// fp32 (ab, aa, bb) of one 16-byte piece: 8 bf16 or 4 fp32 values.
template <bool BF16>
__device__ __forceinline__ void piece_sums(const u32x4& x, const u32x4& y, float& ab, float& aa, float& bb) {
  ab = aa = bb = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (BF16) {
      const float x0 = __uint_as_float(x[e] << 16), x1 = __uint_as_float(x[e] & 0xffff0000u);
      const float y0 = __uint_as_float(y[e] << 16), y1 = __uint_as_float(y[e] & 0xffff0000u);
      ab = fmaf(x0, y0, fmaf(x1, y1, ab));
      aa = fmaf(x0, x0, fmaf(x1, x1, aa));
      bb = fmaf(y0, y0, fmaf(y1, y1, bb));
    } else {
      const float x0 = __uint_as_float(x[e]), y0 = __uint_as_float(y[e]);
      ab = fmaf(x0, y0, ab);
      aa = fmaf(x0, x0, aa);
      bb = fmaf(y0, y0, bb);
    }
  }
}

// Block-wide fp64 sum; every thread gets the total.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) t += red[i];
  return t;
}

// Grid: (n_slabs of one kind, 2): y = 0 keys, 1 values.  VEC: every slab
// starts 16-byte aligned and holds a whole number of 16-byte pieces.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kThreads)
kv_cosine_kernel(const void* k_a, const void* v_a, const void* k_b, const void* v_b, int64_t n_slabs,
                 int64_t slab_elems, float* __restrict__ out) {
  __shared__ double red[kThreads / 64];
  const int64_t s = blockIdx.x;
  const int kv = blockIdx.y;
  const int es = BF16 ? 2 : 4;
  const int64_t off = s * slab_elems * es;
  const char* pa = (const char*)(kv ? v_a : k_a) + off;
  const char* pb = (const char*)(kv ? v_b : k_b) + off;
  double dab = 0.0, daa = 0.0, dbb = 0.0;
  if constexpr (VEC) {
    const uint32_t bytes = (uint32_t)(slab_elems * es);
    const rsrc_t ra = slab_rsrc(pa, bytes), rb = slab_rsrc(pb, bytes);
    const uint32_t step = kThreads * 16 * kUnroll;
    for (uint32_t base = 0; base < bytes; base += step) {
      u32x4 x[kUnroll], y[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        // (a piece past the descriptor reads zeros)
        const uint32_t o = base + (uint32_t)(u * kThreads + threadIdx.x) * 16u;
        x[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, o, 0, 0);
        y[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, o, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float ab, aa, bb;
        piece_sums<BF16>(x[u], y[u], ab, aa, bb);
        dab += ab;
        daa += aa;
        dbb += bb;
      }
    }
  } else {
    for (int64_t e = threadIdx.x; e < slab_elems; e += kThreads) {
      float x, y;
      if constexpr (BF16) {
        x = __uint_as_float((uint32_t)((const uint16_t*)pa)[e] << 16);
        y = __uint_as_float((uint32_t)((const uint16_t*)pb)[e] << 16);
      } else {
        x = ((const float*)pa)[e];
        y = ((const float*)pb)[e];
      }
      dab += (double)x * y;
      daa += (double)x * x;
      dbb += (double)y * y;
    }
  }
  const double ab = block_sum(dab, red);
  const double aa = block_sum(daa, red);
  const double bb = block_sum(dbb, red);
  if (threadIdx.x == 0) out[kv * n_slabs + s] = (float)(ab / (sqrt(aa) * sqrt(bb)));
}

}  // namespace

hipError_t launch_kv_cosine(const void* k_a, const void* v_a, const void* k_b, const void* v_b, int64_t n_slabs,
                            int64_t slab_elems, Dtype dt, float* out, hipStream_t stream) {
  if (n_slabs <= 0) return hipSuccess;
  if (n_slabs > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t es = dt == Dtype::BF16 ? 2 : 4;
  const int64_t bytes = slab_elems * es;
  auto al = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
  const bool vec = bytes % 16 == 0 && bytes <= (int64_t)kMaxSlabBytes && al(k_a) && al(v_a) && al(k_b) && al(v_b);
  const dim3 g((unsigned)n_slabs, 2), b(kThreads);
  if (dt == Dtype::BF16) {
    if (vec)
      hipLaunchKernelGGL((kv_cosine_kernel<true, true>), g, b, 0, stream, k_a, v_a, k_b, v_b, n_slabs, slab_elems, out);
    else
      hipLaunchKernelGGL((kv_cosine_kernel<true, false>), g, b, 0, stream, k_a, v_a, k_b, v_b, n_slabs, slab_elems, out);
  } else {
    if (vec)
      hipLaunchKernelGGL((kv_cosine_kernel<false, true>), g, b, 0, stream, k_a, v_a, k_b, v_b, n_slabs, slab_elems, out);
    else
      hipLaunchKernelGGL((kv_cosine_kernel<false, false>), g, b, 0, stream, k_a, v_a, k_b, v_b, n_slabs, slab_elems, out);
  }
  return hipGetLastError();
}

}  // namespace helm
