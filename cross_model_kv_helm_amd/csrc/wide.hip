// wide.hip — the wide-input map (the Qwen3 cache-mapping write-up, section
// "A linear bridge, strangely enough, suffices": the full mapper's x
// concatenates the KV features of all selected source layers, and every
// target head has its own fits, one for keys and one for values).
//
// Per target layer l and token t the input is
//   x[((j*2 + kv)*H + g)*D + d] = kv == 0 ? (R(-src_pos[t]) src_k[sel_j, g, t, :])[d]
//                                         : src_v[sel_j, g, t, d]
// (IN = k*2*H*D features: selected layer j in layer_sel row order, keys
// before values, source head g), and for every target head h
//   out_k[l, h, t, :] = R(+tgt_pos[t]) (x W_k[l, h] + b_k[l, h]),
//   out_v[l, h, t, :] = x W_v[l, h] + b_v[l, h].
// So each target layer is one dense product [T, IN] x [IN, 2*H*D]: bound by
// the matrix cores (C3 at IN = 8192: 70 TFLOP over ~60 GB of traffic).
//
// Design for MI355X:
//   * Two streaming pre-passes put both operands in k-contiguous bf16, the
//     form the matrix instruction reads: the source keys un-rotated once at
//     src_pos (fp32 arithmetic, rounded once to bf16 — the map's operand
//     type) and each map's W transposed to [D][IN].  Both are HBM-bound and
//     small next to the product (~2 ms of ~40).
//   * Product: v_mfma_f32_32x32x16_bf16, one 256-thread workgroup per
//     256-token x 256-column tile (two (head, K|V) maps), four waves of
//     128 x 128 each (4 x 4 accumulator blocks, 256 fp32 accumulators per
//     lane).  A wave's 128 columns are one whole map, so the RoPE partners
//     d and d+64 sit in the same lane of blocks nb and nb+2.
//   * Operand tiles of 64 k-values reach LDS by buffer->LDS DMA (16 bytes
//     per lane, no registers in between), double-buffered: the copies of
//     step s+1 fly while step s multiplies.  A lane chooses which 16-byte
//     piece it copies, so the tiles are stored XOR-swizzled (piece c of row
//     r at slot r*8 + (c ^ ((r/2) & 7))) and every 16-byte fragment read of
//     the products is bank-conflict free.
//   * XCD-aware tile order: the 8 column tiles of a token tile run on one
//     XCD (workgroup id mod 8), so its activation tile is fetched into that
//     XCD's L2 once and served to all 8.
//   * Epilogue from registers: bias, the forward rotation at tgt_pos (keys;
//     fp32 tables from the RoPE table kernel), round to bf16, store.
#include "internal.hpp"

namespace helm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_void_t;

constexpr int kD = 128;
constexpr int kHalf = 64;
constexpr int kTT = 256;          // tokens per tile
constexpr int kCT = 256;          // output columns per tile (two maps)
constexpr int kKB = 64;           // k-values per pipeline step
constexpr int kThreads = 256;     // four waves, 2 x 2
constexpr int kRowPieces = kKB * 2 / 16;   // 16-byte pieces per tile row and step (8)
constexpr uint32_t kSkip = 0xffffff00u;    // offset past every descriptor: zero load

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Buffer -> LDS copy of 16 bytes per lane: lane i reads the 16 bytes at
// byte offset voff (per lane) of the buffer `rsrc` and they land at
// lds_base + 16*i.  rsrc and lds_base are wave-uniform.  Inline assembly so
// that the compiler does not make later LDS accesses wait for the copy; the
// kernel waits for its copies itself (wait_vmcnt) before the barrier that
// publishes a tile.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, const void* lds_base) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void_t)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(m)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_vmcnt0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0); lgkm and exp untouched
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16-byte slot of piece c of tile row r (XOR swizzle, see the header).
__device__ __forceinline__ int slot(int r, int c) { return r * kRowPieces + (c ^ ((r >> 1) & 7)); }

struct WideArgs {
  const uint16_t* U;          // un-rotated keys [L_s, H, T, D] bf16
  const uint16_t* V;          // values [L_s, H, T, D] bf16
  const uint16_t* WT_k;       // [L_t, H, D, IN] bf16
  const uint16_t* WT_v;
  const float* b_k;           // [L_t, H, D]
  const float* b_v;
  const float2* rope_tgt;     // (cos, sin) at tgt_pos (rope_index layout)
  const int32_t* layer_sel;   // [L_t, k]
  uint16_t* out_k;            // [L_t, H, T, D] bf16
  uint16_t* out_v;
  int32_t L_s, L_t, H, k, T, IN;
  int32_t n_tt, n_ct;         // token tiles, column tiles per target layer
};

__global__ void __launch_bounds__(kThreads, 1) wide_gemm_kernel(WideArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTT * kKB];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kCT * kKB];

  // ---- tile of this workgroup: with token tiles a multiple of 8, the
  // column tiles of one token tile are consecutive on one XCD (id mod 8)
  const int64_t per_layer = (int64_t)a.n_tt * a.n_ct;
  const int32_t l = (int32_t)(blockIdx.x / per_layer);
  const int32_t i = (int32_t)(blockIdx.x % per_layer);
  int32_t tt, ct;
  if (a.n_tt % 8 == 0) {
    const int32_t q = i / 8;
    tt = i % 8 + 8 * (q / a.n_ct);
    ct = q % a.n_ct;
  } else {
    tt = i / a.n_ct;
    ct = i % a.n_ct;
  }
  // an out-of-range selected layer leaves the target layer unwritten (and
  // no address is ever formed from it)
  for (int j = 0; j < a.k; ++j) {
    const int32_t sj = a.layer_sel[l * a.k + j];
    if (sj < 0 || sj >= a.L_s) return;   // uniform over the workgroup, before any barrier
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int32_t t0 = tt * kTT;
  const int32_t T = a.T, H = a.H, IN = a.IN;
  const uint32_t slab_bytes = (uint32_t)T * kD * 2;
  const uint32_t map_bytes = (uint32_t)kD * IN * 2;
  const int n_steps = IN / kKB;

  // ---- operand copies of step s into buffer p: wave w copies the A and
  // B instructions i = w, w+4, ..., w+28; instruction i covers tile rows
  // 8i .. 8i+7, lane q the row 8i + q/8 and slot (q % 8) of it, i.e. piece
  // (q % 8) ^ ((row/2) & 7).
  auto copy_step = [&](int s, int p) __attribute__((always_inline)) {
    const int fb = s >> 1, half = s & 1;                 // feature block (j, kv, g) and its half
    const int j = fb / (2 * H), kv = (fb / H) & 1, g = fb % H;
    const int32_t sl = a.layer_sel[l * a.k + j];
    const uint16_t* slab = (kv ? a.V : a.U) + ((int64_t)sl * H + g) * T * kD;
    const u32x4 ra = rsrc_words(slab, slab_bytes);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int ins = w + 4 * n;
      const int r = 8 * ins + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int32_t t = t0 + r;
      const uint32_t off = t < T ? (uint32_t)t * (kD * 2) + half * (kKB * 2) + 16 * c : kSkip;
      dma16(ra, off, (const char*)As[p] + 1024 * ins);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int ins = w + 4 * n;
      const int r = 8 * ins + (lane >> 3);
      const int mi = 2 * ct + (r >> 7);                  // map: kind * H + head (uniform per instruction)
      const int kind = mi / H, h = mi % H;
      const uint16_t* map = (kind ? a.WT_v : a.WT_k) + ((int64_t)l * H + h) * kD * IN;
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const uint32_t off = (uint32_t)(r & (kD - 1)) * IN * 2 + (uint32_t)s * (kKB * 2) + 16 * c;
      dma16(rsrc_words(map, map_bytes), off, (const char*)Bs[p] + 1024 * ins);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};

  copy_step(0, 0);
  wait_vmcnt0();
  lds_barrier();
  for (int s = 0; s < n_steps; ++s) {
    const int p = s & 1;
    if (s + 1 < n_steps) copy_step(s + 1, p ^ 1);
    const uint16_t* A = As[p];
    const uint16_t* B = Bs[p];
#pragma unroll
    for (int ks = 0; ks < kKB / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = *(const bf16x8*)&A[slot(128 * wm + 32 * mb + (lane & 31), c) * 8];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bfr[nb] = *(const bf16x8*)&B[slot(128 * wn + 32 * nb + (lane & 31), c) * 8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    wait_vmcnt0();        // this wave's copies of step s+1
    lds_barrier();        // everyone's copies landed; everyone is done with buffer p
  }

  // ---- epilogue: this wave's map, bias, forward rotation (keys), store.
  // Accumulator register r of block (mb, nb) holds row 8*(r/4) + 4*(lane/32)
  // + r%4 of the block, column lane%32.
  const int mi = 2 * ct + wn;
  const int kind = mi / H, h = mi % H;
  const int64_t grp = (int64_t)l * H + h;
  const float* bias = (kind ? a.b_v : a.b_k) + grp * kD;
  uint16_t* out = (kind ? a.out_v : a.out_k) + grp * T * kD;
  const int col = lane & 31;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int dlo = 32 * nb + col, dhi = dlo + kHalf;
    const float blo = bias[dlo], bhi = bias[dhi];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t t = t0 + 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t >= T) continue;
        float ylo = acc[mb][nb][r] + blo, yhi = acc[mb][nb + 2][r] + bhi;
        if (kind == 0) {
          const float2 cs = a.rope_tgt[rope_index(t, dlo, kHalf)];
          const float olo = fmaf(ylo, cs.x, -(yhi * cs.y));
          const float ohi = fmaf(yhi, cs.x, ylo * cs.y);
          ylo = olo;
          yhi = ohi;
        }
        out[(int64_t)t * kD + dlo] = __builtin_bit_cast(uint16_t, (__bf16)ylo);
        out[(int64_t)t * kD + dhi] = __builtin_bit_cast(uint16_t, (__bf16)yhi);
      }
    }
  }
}

// Keys un-rotated at src_pos and rounded once to bf16: one thread per
// (row, 16-byte piece of the low half), with the matching piece of the high
// half; (cos, sin) from the RoPE tables.
__global__ void __launch_bounds__(256)
unrotate_keys_kernel(const uint16_t* __restrict__ src_k, const float2* __restrict__ rope_src, int64_t rows,
                     int32_t T, uint16_t* __restrict__ U) {
  const int64_t total = rows * 8;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t row = e >> 3;
    const int pc = (int)(e & 7);
    const int32_t t = (int32_t)(row % T);
    const u32x4 lo = *(const u32x4*)(src_k + row * kD + 8 * pc);
    const u32x4 hi = *(const u32x4*)(src_k + row * kD + kHalf + 8 * pc);
    u32x4 olo, ohi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float2 c0 = rope_src[rope_index(t, 8 * pc + 2 * q, kHalf)];
      const float2 c1 = rope_src[rope_index(t, 8 * pc + 2 * q + 1, kHalf)];
      const float l0 = __uint_as_float(lo[q] << 16), l1 = __uint_as_float(lo[q] & 0xffff0000u);
      const float h0 = __uint_as_float(hi[q] << 16), h1 = __uint_as_float(hi[q] & 0xffff0000u);
      // R(-p): (lo, hi) -> (lo c + hi s, hi c - lo s)
      olo[q] = pack_bf16(fmaf(l0, c0.x, h0 * c0.y), fmaf(l1, c1.x, h1 * c1.y));
      ohi[q] = pack_bf16(fmaf(h0, c0.x, -(l0 * c0.y)), fmaf(h1, c1.x, -(l1 * c1.y)));
    }
    *(u32x4*)(U + row * kD + 8 * pc) = olo;
    *(u32x4*)(U + row * kD + kHalf + 8 * pc) = ohi;
  }
}

// W [G, IN, D] -> WT [G, D, IN] through a 64 x 64 LDS tile per block:
// grid (IN / 64, D / 64, G).
__global__ void __launch_bounds__(256)
transpose_w_kernel(const uint16_t* __restrict__ W, int32_t IN, uint16_t* __restrict__ WT) {
  __shared__ uint16_t tile[64][66];
  const int64_t g = blockIdx.z;
  const int m0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const uint16_t* src = W + g * (int64_t)IN * kD;
  uint16_t* dst = WT + g * (int64_t)kD * IN;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) tile[r][tx] = src[(int64_t)(m0 + r) * kD + d0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4) dst[(int64_t)(d0 + r) * IN + m0 + tx] = tile[tx][r];
}

int grid_for(int64_t work) {
  const int64_t blocks = (work + 255) / 256;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

int64_t wide_in_features(int32_t k, int32_t H, int32_t D) { return (int64_t)k * 2 * H * D; }

bool wide_supports(const WideXfer& x) {
  auto al = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
  const int64_t IN = wide_in_features(x.k, x.H, x.D);
  return x.D == kD && IN % kKB == 0 && (int64_t)x.T * kD * 2 <= 0xffffff00LL && (int64_t)kD * IN * 2 <= 0xffffff00LL &&
         al(x.src_k) && al(x.src_v) && al(x.U) && al(x.WT_k) && al(x.WT_v);
}

hipError_t launch_wide(const WideXfer& x, hipStream_t stream) {
  if (!wide_supports(x)) return hipErrorNotSupported;
  if (x.T <= 0) return hipSuccess;
  const int32_t IN = (int32_t)wide_in_features(x.k, x.H, x.D);
  // pre-pass 1: un-rotated keys of every source layer
  const int64_t rows = (int64_t)x.L_s * x.H * x.T;
  hipLaunchKernelGGL(unrotate_keys_kernel, dim3(grid_for(rows * 8)), dim3(256), 0, stream,
                     (const uint16_t*)x.src_k, x.rope_src, rows, x.T, x.U);
  // pre-pass 2: every map's W transposed to [D, IN]
  const int64_t G = (int64_t)x.L_t * x.H;
  if (G > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_w_kernel, dim3(IN / 64, kD / 64, (unsigned)G), dim3(256), 0, stream,
                     (const uint16_t*)x.W_k, IN, x.WT_k);
  hipLaunchKernelGGL(transpose_w_kernel, dim3(IN / 64, kD / 64, (unsigned)G), dim3(256), 0, stream,
                     (const uint16_t*)x.W_v, IN, x.WT_v);
  // the product with its epilogue
  WideArgs a{};
  a.U = x.U;
  a.V = (const uint16_t*)x.src_v;
  a.WT_k = x.WT_k;
  a.WT_v = x.WT_v;
  a.b_k = x.b_k;
  a.b_v = x.b_v;
  a.rope_tgt = x.rope_tgt;
  a.layer_sel = x.layer_sel;
  a.out_k = (uint16_t*)x.out_k;
  a.out_v = (uint16_t*)x.out_v;
  a.L_s = x.L_s;
  a.L_t = x.L_t;
  a.H = x.H;
  a.k = x.k;
  a.T = x.T;
  a.IN = IN;
  a.n_tt = (x.T + kTT - 1) / kTT;
  a.n_ct = (2 * x.H * kD) / kCT;   // = H
  const int64_t grid = (int64_t)x.L_t * a.n_tt * a.n_ct;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wide_gemm_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace helm
