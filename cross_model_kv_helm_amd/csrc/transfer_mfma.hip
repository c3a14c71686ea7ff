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
//             (v_mfma_f32_32x32x16_bf16), computed as Y^T = W^T X^T so that
//             a lane's accumulators hold 4 consecutive output columns;
//   epilogue  + b, then for keys the forward rotation R(+p') at tgt_pos —
//             always applied — and a nearest-even store to bf16.
//
// Design for MI355X:
//   * Matrix instruction v_mfma_f32_32x32x16_bf16: it sustains its full rate
//     from a single accumulator chain.  Each wave owns one 32-row block of
//     Y^T: rows 0..15 are output columns 16q..16q+15 and rows 16..31 are
//     columns 64+16q..64+16q+15 (q = wave within its group).  In the 32x32
//     accumulator layout rows r and r+16 live in the same lane, so the RoPE
//     partners n and n+64 meet in one lane and the rotation needs no
//     exchange.  W stays in registers (128 VGPRs per wave for k = 4).
//   * Ping-pong.  One workgroup of 8 waves per CU holds two groups: A (waves
//     0-3) and B (waves 4-7); waves w and w+4 share a SIMD.  In every phase
//     one group runs its matrix products and epilogue for a 32-token tile
//     while the other group un-rotates the next tile into LDS, then they swap
//     at a barrier.  So on each SIMD the matrix pipe of one wave overlaps the
//     vector ALU work of the other.
//   * Register prefetch.  Before its matrix products a wave issues the
//     global loads of the source rows of its next un-rotation; they land
//     during its products, epilogue and the other group's phase.
//   * No hidden waits.  gfx9 counts outstanding global loads and stores in
//     one in-order counter, so a wait for any one result also waits for
//     everything issued before it.  Every global access of the tile loop is
//     therefore issued unconditionally (tokens outside the range get a byte
//     offset beyond the descriptor, which the hardware turns into a zero
//     load or a dropped store), and the paged row maps are loaded one phase
//     before they are used: the only waits left are for data that has had a
//     whole phase to arrive.
//   * Persistent sweep over tokens.  Work items are (token chunk, pair of
//     target layers, head, K|V); a workgroup maps all tokens of its item, so W
//     is read from HBM once per item.
//   * XCD-aware order.  Workgroups are dispatched round-robin over the 8
//     XCDs (id mod 8); with the head as the fastest-varying coordinate of the
//     item index and 8 heads, every workgroup of an XCD works on the same
//     head.  All 64 target layers of that head sweep the same tokens at about
//     the same time, so a source row is fetched from HBM once and then served
//     from that XCD's L2 to the ~6 target layers that select it.
//   * Stores through LDS: the epilogue writes its 32x32 block into the
//     group's LDS output tile; in the group's next phase each wave stores
//     whole 256-byte token rows (16 bytes per lane), so every store touches
//     full cache lines.  The tile's (cos, sin) tables use a tile-blocked
//     layout for the same reason: each 16-byte load of a wave is contiguous.
//   * Buffer descriptors.  Source rows, cos/sin tables and output rows are
//     addressed through 128-bit buffer descriptors whose bases are uniform
//     (per layer and head) and live in scalar registers; a lane carries one
//     32-bit byte offset.  The descriptors' record counts also make the
//     hardware drop any access outside the tensor.
#include "internal.hpp"

#include <type_traits>

namespace helm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kD = 128;          // head dimension
constexpr int kHalf = 64;
constexpr int kThreads = 512;    // 8 waves: groups A (0-3) and B (4-7)
constexpr int kGroupThreads = 256;
constexpr int kTile = 32;        // tokens per tile = MFMA B-block width
constexpr int kStageRows = 64;   // W rows staged per pass
constexpr int kStageRow = kStageRows + 8;  // W^T staging row (padded)
constexpr int kCtRow = kHalf + 2;          // staged target (cos, sin) row: 64 float2 + pad
constexpr int kOtRow = kD + 8;             // staged output row: 128 bf16 + pad
constexpr int kRowBytes = kD * 2;          // one bf16 head row
constexpr int kCsTileBytes = kTile * kHalf * 8;   // one tile's (cos, sin) block (rope_index layout)
// Byte offset of a skipped token's row: beyond every descriptor's record
// count (descriptors are limited to kMaxRange bytes), so its loads return
// zero and its stores are dropped.  Adding a row's in-row offset (< 256)
// cannot wrap.
constexpr uint32_t kMaxRange = 0xffffff00u;
constexpr uint32_t kSkipRow = 0xffffff00u;

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;   // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroup barrier that orders LDS accesses only.  The barriers of this
// kernel hand LDS tiles between waves; no wave reads another's global
// stores, so outstanding global loads and stores may stay in flight across
// it (a full __syncthreads() would wait for all of them every phase).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer over [base, base + bytes); accesses beyond it read 0 / are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int KSEL>
struct Cfg {
  static constexpr int KD = KSEL * kD;          // GEMM depth
  static constexpr int KSTEPS = KD / 16;        // 32x32x16 MFMA steps
  static constexpr int ROW = KD + 8;            // LDS row: one token, padded by 16 bytes
  static constexpr int TILE_ELEMS = kTile * ROW;
  // a group's LDS buffer holds its activation tile, and before that the W^T
  // staging block (kD rows of kStageRow)
  static constexpr int BUF_ELEMS = TILE_ELEMS > kD * kStageRow ? TILE_ELEMS : kD * kStageRow;
};

template <int KSEL>
__device__ __forceinline__ int lds_off(int t, int c) {
  return t * Cfg<KSEL>::ROW + (c << 3);
}

// What one thread prefetches for its share of a tile's un-rotation: 16-byte
// chunks pc (low half) and pc+8 (high half) of token pt for each selected
// layer.
template <int KSEL>
struct Raw {
  u32x4 lo[KSEL], hi[KSEL];
  int32_t row;        // paged: source slot of this thread's token of the next tile to load
};

typedef __attribute__((address_space(3))) void* lds_void_t;

// Copies 16 bytes per lane from a buffer into LDS (buffer->LDS DMA): lane
// i reads the 16 bytes at byte offset soff + 16*i of the buffer described by
// `rsrc` and they land at lds_base + 16*i, so one wave moves 1 KB with no
// registers in between.  rsrc, soff and lds_base are wave-uniform.  Written
// as inline assembly on purpose: the compiler cannot tell which LDS buffer a
// copy targets and would otherwise make every later LDS access of the wave
// wait for all outstanding global loads.  The kernel orders these copies
// itself: the issuing wave waits (wait_vmcnt) before the barrier that
// publishes the buffer, and no wave touches a buffer while a copy into it is
// pending.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t soff, const void* lds_base, uint32_t lane16) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void_t)lds_base;
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(lane16), "s"(rsrc), "s"(soff), "s"(m)
               : "memory", "m0");
}

// Plain buffer descriptor words for [base, base + bytes): the same fields
// as make_rsrc, for use as an inline-assembly operand.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Waits until at most N of this wave's global loads, stores and
// global->LDS copies are outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

template <int KSEL, bool PAGED>
__global__ void __launch_bounds__(kThreads, 1)
transfer_mfma_kernel(XferArgs a, int32_t n_pairs, int32_t chunk_tokens, int32_t n_items) {
  using C = Cfg<KSEL>;
  __shared__ __attribute__((aligned(16))) __bf16 xs[2][C::BUF_ELEMS];    // one buffer per group
  __shared__ __attribute__((aligned(16))) float bias_s[2][kD];
  __shared__ __attribute__((aligned(16))) __bf16 ot_s[2][kTile * kOtRow];    // one output tile per group
  // (cos, sin) blocks of a tile in the tile-blocked table layout, by tile
  // parity: source side for the un-rotation, target side for the epilogue
  __shared__ __attribute__((aligned(16))) float2 cs_s[2][kTile * kHalf];
  __shared__ __attribute__((aligned(16))) float2 ct_s[2][kTile * kHalf];

  const int tid = threadIdx.x;
  // group (0 = A, 1 = B) and wave within the group are wave-uniform
  const int gi = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wq = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  const int gtid = tid & 255;
  const int lane = tid & 63;
  const int lr = lane & 31;                // MFMA A row / B column of this lane
  const int lk = lane >> 5;                // MFMA k-half of this lane
  const int wcol = 16 * wq;
  const int my_col = lr < 16 ? wcol + lr : kHalf + wcol + (lr - 16);
  const int pt = gtid >> 3;                // un-rotation share: token of the tile
  const int pc = gtid & 7;                 //   and 16-byte chunk of the low half
  // byte offset of this lane's first epilogue (cos, sin) piece in a tile's
  // target-side table block: piece e = 2lk of chunk 2wq, token lr
  const int ep_off = 2 * lk * (kCsTileBytes / 4) + 128 * lr + 32 * wq;
  __bf16* xg = xs[gi];
  const int LP = (a.L_t + 1) / 2;
  const int32_t n_tok = (int32_t)a.n_tok;
  const uint32_t src_tok_b = (uint32_t)a.src_tok * 2, dst_tok_b = (uint32_t)a.dst_tok * 2;
  const uint32_t src_bytes = (uint32_t)((a.src_rows - 1) * a.src_tok * 2 + kRowBytes);
  const uint32_t dst_bytes = (uint32_t)((a.dst_rows - 1) * a.dst_tok * 2 + kRowBytes);
  const uint32_t tab_bytes = (uint32_t)((a.n_tok + kTile - 1) / kTile * kCsTileBytes);
  const u32x4 tab_src = rsrc_words(a.rope_src, tab_bytes), tab_tgt = rsrc_words(a.rope_tgt, tab_bytes);

  for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int32_t pr = item % n_pairs;
    const int32_t chunk = item / n_pairs;
    const int32_t h = pr % a.H;
    const int32_t rest = pr / a.H;
    const bool keys = rest < LP;           // pairs [0, LP*H) are keys, the rest values
    const int32_t l = 2 * (rest % LP) + gi;
    const int32_t t_begin = chunk * chunk_tokens;   // a multiple of kTile
    const int32_t t_end = min(t_begin + chunk_tokens, n_tok);
    const int nt = (t_end - t_begin + kTile - 1) / kTile;
    const int32_t blk0 = t_begin / kTile;  // table block of the item's first tile

    // this group's selected source layers; a missing target layer (odd L_t)
    // or an out-of-range entry makes the group idle (it still meets barriers)
    bool active = l < a.L_t;
    rsrc_t srs[KSEL];
#pragma unroll
    for (int j = 0; j < KSEL; ++j) {
      const int32_t sj = active ? a.layer_sel[l * KSEL + j] : 0;
      active = active && sj >= 0 && sj < a.L_s;
      const uint16_t* base = (const uint16_t*)(keys ? a.src_k : a.src_v) +
                             (active ? (int64_t)sj * a.src_layer + (int64_t)h * a.src_head : 0);
      srs[j] = make_rsrc(base, src_bytes);
    }
    const int32_t grp = (active ? l : 0) * a.H + h;
    const uint16_t* W = (const uint16_t*)(keys ? a.W_k : a.W_v) + (int64_t)grp * C::KD * kD;
    const float* bias = (keys ? a.b_k : a.b_v) + (int64_t)grp * kD;
    const rsrc_t dst = make_rsrc((const uint16_t*)(keys ? a.out_k : a.out_v) +
                                     (active ? (int64_t)l * a.dst_layer + (int64_t)h * a.dst_head : 0),
                                 dst_bytes);

    // ---- W^T fragments of this wave's 32 columns, in registers: lane holds
    // W[m = 16s + 8*lk + i][my_col], i < 8.  W is staged through this
    // group's LDS tile 64 rows at a time, transposed on the way in
    // (coalesced 16-byte global loads, 2-byte LDS stores), so that each
    // fragment is one 16-byte LDS read.
    bf16x8 wf[C::KSTEPS];
#pragma unroll
    for (int part = 0; part < C::KD / kStageRows; ++part) {
      lds_barrier();                                 // earlier readers of xs are done
      if (active) {
        const u32x4* gsrc = (const u32x4*)(W + (int64_t)part * kStageRows * kD);
#pragma unroll 2
        for (int e = gtid; e < kStageRows * kD / 8; e += kGroupThreads) {
          const u32x4 v = gsrc[e];
          const int m = e >> 4, n0 = (e & 15) << 3;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            xg[(n0 + 2 * q) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] & 0xffffu));
            xg[(n0 + 2 * q + 1) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] >> 16));
          }
        }
      }
      lds_barrier();
      if (active) {
#pragma unroll
        for (int s4 = 0; s4 < kStageRows / 16; ++s4)
          wf[(kStageRows / 16) * part + s4] = *(const bf16x8*)&xg[my_col * kStageRow + 16 * s4 + 8 * lk];
      }
    }
    if (active && gtid < kD / 4) ((float4*)bias_s[gi])[gtid] = ((const float4*)bias)[gtid];

    int32_t drow[2] = {0, 0};   // paged: target slots of the rows this thread stores next

    // ---- per-thread pieces of the tile pipeline
    // Issues the loads of tile `tile`'s source rows (this thread's token pt,
    // chunks pc and pc+8 of each selected layer).  Skipped tokens load zeros.
    auto load_raw = [&](int tile, Raw<KSEL>& r) __attribute__((always_inline)) {
      const int32_t n = t_begin + tile * kTile + pt;
      const bool ok = tile < nt && n < t_end;
      uint32_t rowb;
      if constexpr (PAGED) {
        rowb = ok && r.row >= 0 ? (uint32_t)r.row * src_tok_b : kSkipRow;
        // slot of the token one tile later, used by the next call
        r.row = a.src_row[min(n + kTile, t_end - 1)];
      } else {
        rowb = ok ? (uint32_t)n * src_tok_b : kSkipRow;
      }
      const uint32_t off = rowb + 16 * pc;
#pragma unroll
      for (int j = 0; j < KSEL; ++j) {
        r.lo[j] = __builtin_amdgcn_raw_buffer_load_b128(srs[j], off, 0, 0);
        r.hi[j] = __builtin_amdgcn_raw_buffer_load_b128(srs[j], off + kHalf * 2, 0, 0);
      }
    };
    // One of the four 1 KB pieces that this wave copies of a tile's (cos,
    // sin) block (keys only): piece q of wave wq is bytes [(4q + wq) KB, +1 KB).
    auto table_piece = [&](const u32x4& table, float2* dst, int tile, int q) __attribute__((always_inline)) {
      if (keys && tile < nt) {
        const uint32_t off = (4 * q + wq) * 1024;
        dma16(table, (uint32_t)(blk0 + tile) * kCsTileBytes + off, (char*)dst + off, 16 * lane);
      }
    };
    // Un-rotates (keys) the loaded rows and writes them into the group's
    // activation tile.  A skipped token's row is zero in, and whatever it
    // becomes only reaches its own output column, which is never stored.
    auto store_tile = [&](Raw<KSEL>& r, const float2* cs_tab) __attribute__((always_inline)) {
      if (keys) {
        // tile-blocked table: piece e of (token pt, chunk pc) at e*4KB + pt*128 + pc*16
        f32x4 cs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cs[e] = *(const f32x4*)((const char*)cs_tab + e * (kCsTileBytes / 4) + 128 * pt + 16 * pc);
        // one layer at a time, so only one layer's values are unpacked to fp32
#pragma unroll
        for (int j = 0; j < KSEL; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4 v = cs[e];    // (cos, sin) of dims 8pc+2e and 8pc+2e+1
            const float l0 = bf16lo(r.lo[j][e]), l1 = bf16hi(r.lo[j][e]);
            const float h0 = bf16lo(r.hi[j][e]), h1 = bf16hi(r.hi[j][e]);
            // R(-p): (lo, hi) -> (lo c + hi s, hi c - lo s)
            r.lo[j][e] = pack_bf16(fmaf(l0, v.x, h0 * v.y), fmaf(l1, v.z, h1 * v.w));
            r.hi[j][e] = pack_bf16(fmaf(h0, v.x, -(l0 * v.y)), fmaf(h1, v.z, -(l1 * v.w)));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int j = 0; j < KSEL; ++j) {
        *(u32x4*)&xg[lds_off<KSEL>(pt, 16 * j + pc)] = r.lo[j];
        *(u32x4*)&xg[lds_off<KSEL>(pt, 16 * j + 8 + pc)] = r.hi[j];
      }
    };
    // Writes a computed tile from this group's LDS output tile to the target
    // cache: 16 threads per token row, 16 bytes each, so a wave stores whole
    // 256-byte rows.  Always exactly two stores per thread.
    auto store_out = [&](int tile) __attribute__((always_inline)) {
      const int seg = gtid & 15;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = (gtid >> 4) + 16 * hh;
        const int32_t n = t_begin + tile * kTile + r;
        const int32_t row = PAGED ? drow[hh] : n;
        const uint32_t rowb = n < t_end && row >= 0 ? (uint32_t)row * dst_tok_b : kSkipRow;
        const u32x4 v = *(const u32x4*)&ot_s[gi][r * kOtRow + 8 * seg];
        __builtin_amdgcn_raw_buffer_store_b128(v, dst, rowb + 16 * seg, 0, 0);
      }
    };
    // Matrix products Y^T = W^T X^T of tile `tile`, bias, forward rotation
    // into the LDS output tile.  The global loads of the group's next
    // un-rotation are issued first; with CS_DMA (group A) the copy of the
    // next tile's source-side table is spread over the first products.
    // Ends with every global access of this wave complete.
    auto compute_tile = [&](int tile, Raw<KSEL>& raw, auto cs_dma) __attribute__((always_inline)) {
      constexpr bool CS_DMA = decltype(cs_dma)::value;
      float2* cs_next = cs_s[(tile + 1) & 1];
      if (!active) {
        if constexpr (CS_DMA) {
#pragma unroll
          for (int q = 0; q < 4; ++q) table_piece(tab_src, cs_next, tile + 1, q);
        }
        wait_vmcnt<0>();
        return;
      }
      const float2* ct_tab = ct_s[tile & 1];
      if constexpr (PAGED) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          drow[hh] = a.dst_row[min(t_begin + tile * kTile + (gtid >> 4) + 16 * hh, t_end - 1)];
      }
      load_raw(tile + 1, raw);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int kAhead = KSEL <= 2 ? C::KSTEPS : 4;   // LDS fragments read ahead
      // step after whose product the epilogue's LDS reads are issued (with
      // k >= 3 there are no registers to hold them during the products)
      constexpr int kEpi = KSEL <= 2 ? C::KSTEPS - 4 : C::KSTEPS - 1;
      f32x16 acc = {};
      bf16x8 xf[kAhead];
      float4 eb[4], ec[4];   // bias and (cos, sin) for the epilogue
#pragma unroll
      for (int s = 0; s < kAhead; ++s) xf[s] = *(const bf16x8*)&xg[lds_off<KSEL>(lr, 2 * s + lk)];
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], xf[s % kAhead], acc, 0, 0, 0);
        if (s + kAhead < C::KSTEPS) xf[s % kAhead] = *(const bf16x8*)&xg[lds_off<KSEL>(lr, 2 * (s + kAhead) + lk)];
        if constexpr (CS_DMA) {
          if (s < 4) table_piece(tab_src, cs_next, tile + 1, s);
        }
        if (s == kEpi) {
          // columns c0 = wcol + 8g + 4lk .. c0+3 of token lr are table
          // pieces e = 2lk and 2lk+1 of chunk 2wq + g (tile-blocked layout)
          const char* tb = (const char*)ct_tab + ep_off;
          const float* bb = &bias_s[gi][wcol + 4 * lk];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            eb[2 * g] = *(const float4*)(bb + 8 * g);
            eb[2 * g + 1] = *(const float4*)(bb + 8 * g + kHalf);
            if (keys) {
              ec[2 * g] = *(const float4*)(tb + 16 * g);
              ec[2 * g + 1] = *(const float4*)(tb + 16 * g + kCsTileBytes / 4);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // epilogue.  Accumulator j < 8 is column wcol + 8*(j/4) + 4*lk + j%4
      // of token lr; j + 8 is its partner 64 columns up.
      __bf16* ot = ot_s[gi];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int c0 = wcol + 8 * g + 4 * lk;
        const float4 bl = eb[2 * g], bh = eb[2 * g + 1];
        float y0[4] = {acc[4 * g] + bl.x, acc[4 * g + 1] + bl.y, acc[4 * g + 2] + bl.z, acc[4 * g + 3] + bl.w};
        float y1[4] = {acc[8 + 4 * g] + bh.x, acc[9 + 4 * g] + bh.y, acc[10 + 4 * g] + bh.z,
                       acc[11 + 4 * g] + bh.w};
        if (keys) {
          const float4 v0 = ec[2 * g], v1 = ec[2 * g + 1];
          const float cc[4] = {v0.x, v0.z, v1.x, v1.z};
          const float ss[4] = {v0.y, v0.w, v1.y, v1.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // R(+p'): (lo, hi) -> (lo c - hi s, hi c + lo s)
            const float o0 = fmaf(y0[j], cc[j], -(y1[j] * ss[j]));
            const float o1 = fmaf(y1[j], cc[j], y0[j] * ss[j]);
            y0[j] = o0;
            y1[j] = o1;
          }
        }
        *(uint2*)&ot[lr * kOtRow + c0] = make_uint2(pack_bf16(y0[0], y0[1]), pack_bf16(y0[2], y0[3]));
        *(uint2*)&ot[lr * kOtRow + c0 + kHalf] = make_uint2(pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3]));
      }
      wait_vmcnt<0>();
    };

    // ---- ping-pong over tiles.  Phase 2i: A computes tile i while B
    // un-rotates tile i; phase 2i+1: B computes tile i while A un-rotates
    // tile i+1.  A group stores its previous tile's output at the start of
    // its un-rotation phase.  Group A copies the tables: the source side of
    // tile i+1 during its products of tile i (read from the next phase on)
    // and the target side of tile i+1 during its un-rotation phase (read
    // from the phase after).  Table buffers alternate with the tile parity.
    // Each group runs its own copy of the loop, so every register value has
    // one producer and one consumer; both copies meet the same barriers.
    auto run = [&](auto group) __attribute__((always_inline)) {
      constexpr int G = decltype(group)::value;
      Raw<KSEL> raw;
      if constexpr (PAGED) raw.row = nt > 0 ? a.src_row[t_begin + pt < t_end ? t_begin + pt : t_end - 1] : -1;
      if (active) load_raw(0, raw);
      if constexpr (G == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          table_piece(tab_src, cs_s[0], 0, q);
          table_piece(tab_tgt, ct_s[0], 0, q);
        }
      }
      wait_vmcnt<0>();
      lds_barrier();                                   // bias and the first tables are visible
      if (G == 0 && active) store_tile(raw, cs_s[0]);
      lds_barrier();
      for (int i = 0; i < nt; ++i) {
        if constexpr (G == 0) {
          compute_tile(i, raw, std::integral_constant<bool, true>());
          lds_barrier();
#pragma unroll
          for (int q = 0; q < 4; ++q) table_piece(tab_tgt, ct_s[(i + 1) & 1], i + 1, q);
          if (active) {
            store_out(i);
            if (i + 1 < nt) store_tile(raw, cs_s[(i + 1) & 1]);
          }
          wait_vmcnt<2>();                             // the table copy; the two stores may stay in flight
          lds_barrier();
        } else {
          if (active) {
            if (i > 0) store_out(i - 1);
            store_tile(raw, cs_s[i & 1]);
          }
          lds_barrier();
          compute_tile(i, raw, std::integral_constant<bool, false>());
          lds_barrier();
        }
      }
      if (G == 1 && active && nt > 0) store_out(nt - 1);
    };
    if (gi == 0)
      run(std::integral_constant<int, 0>());
    else
      run(std::integral_constant<int, 1>());
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
  // 16-byte vector loads of source rows, W and bias, 16-byte stores of
  // outputs, and every buffer descriptor's byte range below kMaxRange
  auto al = [](const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; };
  const int64_t lim = kMaxRange;
  const bool ranges = (a.n_tok + kTile - 1) / kTile * kCsTileBytes <= lim &&
                      (a.src_rows - 1) * a.src_tok * 2 + kRowBytes <= lim &&
                      (a.dst_rows - 1) * a.dst_tok * 2 + kRowBytes <= lim && a.n_tok < 0x7fffffffLL;
  return ranges && a.D == kD && a.k >= 1 && a.k <= 4 && al(a.src_k, 16) && al(a.src_v, 16) && al(a.W_k, 16) &&
         al(a.W_v, 16) && al(a.out_k, 16) && al(a.out_v, 16) && al(a.rope_src, 16) && al(a.rope_tgt, 16) &&
         al(a.b_k, 16) && al(a.b_v, 16);
}

hipError_t launch_transfer_mfma(const XferArgs& a, hipStream_t stream) {
  if (!mfma_supports(a)) return hipErrorNotSupported;
  if (a.n_tok <= 0) return hipSuccess;
  const int64_t n_pairs = (int64_t)((a.L_t + 1) / 2) * a.H * 2;
  const int64_t slots = cu_count();   // one 8-wave workgroup per CU
  // Split tokens into chunks only when there are fewer pairs than CUs.
  int64_t n_chunks = 1;
  if (n_pairs < slots) n_chunks = (slots + n_pairs - 1) / n_pairs;
  int64_t chunk_tokens = (a.n_tok + n_chunks - 1) / n_chunks;
  chunk_tokens = (chunk_tokens + kTile - 1) / kTile * kTile;
  n_chunks = (a.n_tok + chunk_tokens - 1) / chunk_tokens;
  const int64_t n_items = n_pairs * n_chunks;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t grid = n_items < slots ? n_items : slots;
  const dim3 g((unsigned)grid), b(kThreads);
  const int32_t np = (int32_t)n_pairs, ct = (int32_t)chunk_tokens, ni = (int32_t)n_items;
  const bool paged = a.src_row != nullptr;
  if (paged != (a.dst_row != nullptr)) return hipErrorInvalidValue;
#define HELM_LAUNCH(K)                                                                  \
  do {                                                                                  \
    if (paged)                                                                          \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, true>), g, b, 0, stream, a, np, ct, ni); \
    else                                                                                \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, false>), g, b, 0, stream, a, np, ct, ni); \
  } while (0)
  switch (a.k) {
    case 1: HELM_LAUNCH(1); break;
    case 2: HELM_LAUNCH(2); break;
    case 3: HELM_LAUNCH(3); break;
    default: HELM_LAUNCH(4); break;
  }
#undef HELM_LAUNCH
  return hipGetLastError();
}

}  // namespace helm
