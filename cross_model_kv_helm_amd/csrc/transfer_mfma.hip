// transfer_mfma.hip — matrix-core transfer kernel for bf16 storage (gfx950).
//
// What it computes is the whole transfer for one (target layer l, head h,
// K|V) group over a range of tokens (pages: "Helm Intelligent Routing",
// section "Why carrying the cache across is the hard part"; the Qwen3
// cache-mapping write-up, section "A linear bridge, strangely enough,
// suffices"):
//   prologue  gather the k selected source layers' rows of head h and, for
//             keys, un-rotate them at src_pos (R(-p)), rounding the content
//             key once to bf16 — the operand type of the map;
//   product   Y = X W on the matrix cores, bf16 x bf16 -> fp32
//             (v_mfma_f32_16x16x32_bf16), computed as Y^T = W^T X^T so that
//             a lane's accumulators hold 4 consecutive output columns;
//   epilogue  + b, then for keys the forward rotation R(+p') at tgt_pos —
//             always applied — and a nearest-even store to bf16.
//
// Design for MI355X:
//   * W stays in registers.  A workgroup (4 waves, one per SIMD) owns one
//     group at a time; wave w holds W[:, cols] for its 32 output columns
//     {16w..16w+15} and {64+16w..64+16w+15} — RoPE partners n and n+64 land
//     in the same lane, so the epilogue rotation needs no data exchange.
//     For k = 4 that is 128 VGPRs per lane; two workgroups share a CU.
//   * Persistent sweep over tokens.  Work items are (token chunk, group); a
//     workgroup maps all tokens of its item in 32-token tiles, so W is read
//     from HBM once per item, not once per tile.
//   * XCD-aware order.  Workgroups are dispatched round-robin over the 8
//     XCDs (id mod 8); with the head as the fastest-varying coordinate of the
//     group index and 8 heads, every workgroup of an XCD works on the same
//     head.  All target layers of that head sweep the same tokens at about
//     the same time, so each source row is fetched from HBM once and then
//     served from that XCD's L2 to the ~6 target layers that select it.
//   * 16-token activation tiles through LDS, double-buffered, one barrier
//     per tile.
//     Rows are padded by 16 bytes so the 16 lanes of a B-operand read hit
//     distinct banks.
#include "internal.hpp"

namespace helm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head dimension
constexpr int kHalf = 64;
constexpr int kThreads = 256;    // 4 waves
constexpr int kTile = 16;        // tokens per tile (one MFMA token block)
constexpr int kTB = kTile / 16;  // MFMA token blocks per tile
constexpr int kStageRow = kD + 8; // W^T staging row: 128 inputs of one output column, padded

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;   // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int KSEL>
struct Cfg {
  static constexpr int KD = KSEL * kD;          // GEMM depth
  static constexpr int KSTEPS = KD / 32;        // 16x16x32 MFMA steps
  static constexpr int ROW = KD + 8;            // LDS row: one token, padded by 16 bytes
  static constexpr int TILE_ELEMS = kTile * ROW;
};

// LDS element offset of chunk `c` (8 bf16) of token row `t`.  The 16-byte
// pad per row puts the 16 rows a B-operand read touches on distinct banks,
// and keeps offsets additive so every k-step uses an immediate offset.
template <int KSEL>
__device__ __forceinline__ int lds_off(int t, int c) {
  return t * Cfg<KSEL>::ROW + (c << 3);
}

template <int KSEL>
__global__ void __launch_bounds__(kThreads, 2)
transfer_mfma_kernel(XferArgs a, int32_t n_groups, int64_t chunk_tokens, int64_t n_items) {
  using C = Cfg<KSEL>;
  // One LDS buffer serves two purposes: the W^T staging block while a group's
  // weights are loaded, then the two activation tiles.
  constexpr int kLdsElems = 2 * C::TILE_ELEMS > kD * kStageRow ? 2 * C::TILE_ELEMS : kD * kStageRow;
  __shared__ __attribute__((aligned(16))) __bf16 lds[kLdsElems];
  __bf16 (*xs)[C::TILE_ELEMS] = reinterpret_cast<__bf16 (*)[C::TILE_ELEMS]>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 15;      // MFMA row/col within a 16-block
  const int lgrp = lane >> 4;      // MFMA k-group (0..3)

  int buf = 0;
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int32_t g = (int32_t)(item % n_groups);
    const int64_t chunk = item / n_groups;
    const int32_t h = g % a.H;
    const int32_t rest = g / a.H;
    const int32_t l = rest % a.L_t;
    const bool keys = rest < a.L_t;    // groups [0, L_t*H) are keys, the rest values
    const int64_t t_begin = chunk * chunk_tokens;
    int64_t t_end = t_begin + chunk_tokens;
    if (t_end > a.n_tok) t_end = a.n_tok;

    // selected source layers; an out-of-range entry skips the whole group
    int32_t sel[KSEL];
    bool valid = true;
#pragma unroll
    for (int j = 0; j < KSEL; ++j) {
      sel[j] = a.layer_sel[(int64_t)l * KSEL + j];
      valid = valid && sel[j] >= 0 && sel[j] < a.L_s;
    }
    if (!valid) continue;   // uniform across the workgroup

    const int32_t grp = l * a.H + h;
    const uint16_t* W = (const uint16_t*)(keys ? a.W_k : a.W_v) + (int64_t)grp * C::KD * kD;
    const float* bias = (keys ? a.b_k : a.b_v) + (int64_t)grp * kD;
    const uint16_t* src = (const uint16_t*)(keys ? a.src_k : a.src_v);
    uint16_t* out = (uint16_t*)(keys ? a.out_k : a.out_v);

    // ---- W^T fragments for this wave's two 16-column blocks, in registers.
    // lane holds W[m = 32s + 8*lgrp + i][n = ncol + lrow], i < 8.  W is
    // staged through LDS one 128-row block at a time, transposed on the way
    // in (coalesced 16-byte global loads, 2-byte LDS stores), so that each
    // fragment is one 16-byte LDS read.
    const int ncol0 = 16 * wave, ncol1 = kHalf + 16 * wave;
    bf16x8 wf[2][C::KSTEPS];
    {
      __bf16* stage = lds;                            // W^T block [kD][kStageRow]
#pragma unroll
      for (int part = 0; part < KSEL; ++part) {
        __syncthreads();                              // earlier readers of the buffer are done
        const u32x4* gsrc = (const u32x4*)(W + (int64_t)part * kD * kD);
#pragma unroll 2
        for (int e = tid; e < kD * kD / 8; e += kThreads) {
          const u32x4 v = gsrc[e];
          const int m = e >> 4, n0 = (e & 15) << 3;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            stage[(n0 + 2 * q) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] & 0xffffu));
            stage[(n0 + 2 * q + 1) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] >> 16));
          }
        }
        __syncthreads();
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int s = 4 * part + s4, m = 32 * s4 + 8 * lgrp;
          wf[0][s] = *(const bf16x8*)&stage[(ncol0 + lrow) * kStageRow + m];
          wf[1][s] = *(const bf16x8*)&stage[(ncol1 + lrow) * kStageRow + m];
        }
      }
      __syncthreads();                                // the buffer is reused by the first tile
    }
    // bias for the 4 columns this lane's accumulators hold in each block
    float b0[4], b1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0[j] = bias[ncol0 + 4 * lgrp + j];
      b1[j] = bias[ncol1 + 4 * lgrp + j];
    }

    // ---- prologue assignment: thread -> (token pt, 16-byte chunk pc of the low
    // half, layer parity pj): it loads dims 8pc.. and 64+8pc.. of layers pj, pj+2, ..
    const int pt = tid >> 4;        // 0..15
    const int pj = (tid >> 3) & 1;
    const int pc = tid & 7;
    constexpr int kMine = (KSEL + 1) / 2;   // layers per thread (upper bound)

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
      // -- gather (+ un-rotate) one tile into xs[buf]
      {
        const int64_t n = t0 + pt;
        u32x4 lo[kMine], hi[kMine];
        bool have = n < t_end;
        int64_t row = 0;
        if (have) {
          row = a.src_row ? (int64_t)a.src_row[n] : n;
          have = row >= 0;
        }
#pragma unroll
        for (int q = 0; q < kMine; ++q) {
          lo[q] = u32x4{0, 0, 0, 0};
          hi[q] = u32x4{0, 0, 0, 0};
        }
        if (have) {
#pragma unroll
          for (int q = 0; q < kMine; ++q) {
            const int j = pj + 2 * q;
            if (j < KSEL) {
              const uint16_t* p = src + (int64_t)sel[j] * a.src_layer + (int64_t)h * a.src_head +
                                  row * a.src_tok + 8 * pc;
              lo[q] = *(const u32x4*)p;
              hi[q] = *(const u32x4*)(p + kHalf);
            }
          }
          if (keys) {
            const float4* cs4 = (const float4*)(a.rope_src + n * kHalf + 8 * pc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float4 v = cs4[e];   // (cos, sin) of dims 8pc+2e and 8pc+2e+1
#pragma unroll
              for (int q = 0; q < kMine; ++q) {
                const float l0 = bf16lo(lo[q][e]), l1 = bf16hi(lo[q][e]);
                const float h0 = bf16lo(hi[q][e]), h1 = bf16hi(hi[q][e]);
                // R(-p): (lo, hi) -> (lo c + hi s, hi c - lo s)
                lo[q][e] = pack_bf16(fmaf(l0, v.x, h0 * v.y), fmaf(l1, v.z, h1 * v.w));
                hi[q][e] = pack_bf16(fmaf(h0, v.x, -(l0 * v.y)), fmaf(h1, v.z, -(l1 * v.w)));
              }
            }
          }
        }
#pragma unroll
        for (int q = 0; q < kMine; ++q) {
          const int j = pj + 2 * q;
          if (j < KSEL) {
            *(u32x4*)&xs[buf][lds_off<KSEL>(pt, 16 * j + pc)] = lo[q];
            *(u32x4*)&xs[buf][lds_off<KSEL>(pt, 16 * j + 8 + pc)] = hi[q];
          }
        }
      }
      __syncthreads();

      // -- Y^T = W^T X^T for this wave's 32 columns x 32 tokens
      f32x4 acc[2][kTB];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) acc[b][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) {
          const int t = 16 * tb + lrow;
          const bf16x8 xf = *(const bf16x8*)&xs[buf][lds_off<KSEL>(t, 4 * s + lgrp)];
          acc[0][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[0][s], xf, acc[0][tb], 0, 0, 0);
          acc[1][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[1][s], xf, acc[1][tb], 0, 0, 0);
        }
      }

      // -- epilogue: bias, forward rotation (keys), store
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const int64_t n = t0 + 16 * tb + lrow;
        if (n >= t_end) continue;
        const int64_t row = a.dst_row ? (int64_t)a.dst_row[n] : n;
        if (row < 0) continue;
        float o0[4], o1[4];
        if (keys) {
          const float4* cs4 = (const float4*)(a.rope_tgt + n * kHalf + ncol0 + 4 * lgrp);
          const float4 v0 = cs4[0], v1 = cs4[1];
          const float c[4] = {v0.x, v0.z, v1.x, v1.z}, s[4] = {v0.y, v0.w, v1.y, v1.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float y0 = acc[0][tb][j] + b0[j], y1 = acc[1][tb][j] + b1[j];
            // R(+p'): (lo, hi) -> (lo c - hi s, hi c + lo s)
            o0[j] = fmaf(y0, c[j], -(y1 * s[j]));
            o1[j] = fmaf(y1, c[j], y0 * s[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            o0[j] = acc[0][tb][j] + b0[j];
            o1[j] = acc[1][tb][j] + b1[j];
          }
        }
        uint16_t* q = out + (int64_t)l * a.dst_layer + (int64_t)h * a.dst_head + row * a.dst_tok;
        uint2 w0, w1;
        w0.x = pack_bf16(o0[0], o0[1]); w0.y = pack_bf16(o0[2], o0[3]);
        w1.x = pack_bf16(o1[0], o1[1]); w1.y = pack_bf16(o1[2], o1[3]);
        *(uint2*)(q + ncol0 + 4 * lgrp) = w0;
        *(uint2*)(q + ncol1 + 4 * lgrp) = w1;
      }
      buf ^= 1;
    }
  }
}

int g_cu_count = 0;

int cu_count() {
  if (g_cu_count == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_cu_count = n;
    else
      g_cu_count = 256;
  }
  return g_cu_count;
}

}  // namespace

bool mfma_supports(const XferArgs& a) {
  // 16-byte vector loads of source rows and W, 8-byte stores of outputs
  auto al = [](const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; };
  return a.D == kD && a.k >= 1 && a.k <= 4 && al(a.src_k, 16) && al(a.src_v, 16) && al(a.W_k, 16) &&
         al(a.W_v, 16) && al(a.out_k, 8) && al(a.out_v, 8) && al(a.rope_src, 16) && al(a.rope_tgt, 16);
}

hipError_t launch_transfer_mfma(const XferArgs& a, hipStream_t stream) {
  if (!mfma_supports(a)) return hipErrorNotSupported;
  if (a.n_tok <= 0) return hipSuccess;
  const int64_t n_groups = (int64_t)a.L_t * a.H * 2;
  const int64_t slots = 2LL * cu_count();   // two workgroups per CU
  // Split tokens into chunks only when there are fewer groups than slots.
  int64_t n_chunks = 1;
  if (n_groups < slots) n_chunks = (slots + n_groups - 1) / n_groups;
  int64_t chunk_tokens = (a.n_tok + n_chunks - 1) / n_chunks;
  chunk_tokens = (chunk_tokens + kTile - 1) / kTile * kTile;
  n_chunks = (a.n_tok + chunk_tokens - 1) / chunk_tokens;
  const int64_t n_items = n_groups * n_chunks;
  const int64_t grid = n_items < slots ? n_items : slots;
  const dim3 g((unsigned)grid), b(kThreads);
  switch (a.k) {
    case 1: hipLaunchKernelGGL(transfer_mfma_kernel<1>, g, b, 0, stream, a, (int32_t)n_groups, chunk_tokens, n_items); break;
    case 2: hipLaunchKernelGGL(transfer_mfma_kernel<2>, g, b, 0, stream, a, (int32_t)n_groups, chunk_tokens, n_items); break;
    case 3: hipLaunchKernelGGL(transfer_mfma_kernel<3>, g, b, 0, stream, a, (int32_t)n_groups, chunk_tokens, n_items); break;
    default: hipLaunchKernelGGL(transfer_mfma_kernel<4>, g, b, 0, stream, a, (int32_t)n_groups, chunk_tokens, n_items); break;
  }
  return hipGetLastError();
}

}  // namespace helm
