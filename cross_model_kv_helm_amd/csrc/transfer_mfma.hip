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
//   * Matrix instruction v_mfma_f32_32x32x16_bf16.  A matrix wave owns one
//     32-row block of Y^T: rows 0..15 are output columns 16q..16q+15 and rows
//     16..31 are columns 64+16q..64+16q+15 (q = wave within its role).  In the
//     32x32 accumulator layout rows r and r+16 live in the same lane, so the
//     RoPE partners n and n+64 meet in one lane and the rotation needs no
//     exchange.  W stays in registers (128 VGPRs per wave for k = 4) for the
//     whole token sweep of an item.
//   * Two roles per CU, one wave of each on every SIMD: four matrix waves
//     (products, epilogue, target-table copies, output stores) and four data
//     waves (source-row loads, un-rotation into LDS).  One LDS barrier ends
//     each 32-token phase; the matrix pipe of one wave overlaps the vector ALU
//     and memory work of the other.
//   * Register prefetch.  The data waves load the source rows of a tile two
//     phases ahead, layer by layer between the un-rotation arithmetic.
//   * Keys and values are separate launches: values have no rotation, so
//     their items issue no table loads or copies.
//   * No hidden waits.  gfx9 counts outstanding global loads and stores in
//     one in-order counter, so a wait for any one result also waits for
//     everything issued before it.  Every global access of the tile loop is
//     therefore issued unconditionally (tokens outside the range get a byte
//     offset beyond the descriptor, which the hardware turns into a zero
//     load or a dropped store), and the paged row maps are loaded one phase
//     before they are used: the only waits left are for data that has had a
//     whole phase to arrive.
//   * Persistent sweep over tokens.  Work items are (token chunk, target
//     layer, head); a workgroup maps all tokens of its item, so W is read
//     from HBM once per item.
//   * XCD-aware order.  Workgroups are dispatched round-robin over the 8
//     XCDs (id mod 8); with the head as the fastest-varying coordinate of the
//     item index and 8 heads, every workgroup of an XCD works on the same
//     head, so the ~3 target layers that select a source row read it from
//     that XCD's L2 at about the same time.
//   * Stores through LDS: the epilogue writes its 32x32 block into an LDS
//     output tile; two phases later each wave stores whole 256-byte token
//     rows (16 bytes per lane), so every store touches full cache lines.  The
//     tile's (cos, sin) tables use a tile-blocked layout for the same reason:
//     each 16-byte load of a wave is contiguous.
//   * Buffer descriptors.  Source rows, cos/sin tables and output rows are
//     addressed through 128-bit buffer descriptors whose bases are uniform
//     (per layer and head) and live in scalar registers; a lane carries one
//     32-bit byte offset.  The descriptors' record counts also make the
//     hardware drop any access outside the tensor.
#include "internal.hpp"

#include <atomic>
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
constexpr int kDepth = 2;        // source-row register sets of a data thread (prefetch depth)
constexpr int kTile = 32;        // tokens per tile = MFMA B-block width
constexpr int kStageRows = 64;   // W rows staged per pass
constexpr int kStageRow = kStageRows + 8;  // W^T staging row (padded)
constexpr int kOtRow = kD + 8;             // staged output row: 128 bf16 + pad
constexpr int kRowBytes = kD * 2;          // one bf16 head row
constexpr int kCsTileBytes = kTile * kHalf * 8;   // one tile's (cos, sin) block (rope_index layout)
// Byte offset of a skipped token's row: beyond every descriptor's record
// count (descriptors are limited to kMaxRange bytes), so its loads return
// zero and its stores are dropped.  Adding a row's in-row offset (< 256)
// cannot wrap.
constexpr uint32_t kMaxRange = 0xffffff00u;
constexpr uint32_t kSkipRow = 0xffffff00u;
constexpr int kStoreNT = 2;      // cache-policy bits of the output stores: nt (streaming)

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
// layer, and the (cos, sin) pairs of dims 8pc .. 8pc+7 of that token.
template <int KSEL>
struct Raw {
  u32x4 lo[KSEL], hi[KSEL];
  f32x4 cs[4];
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

// The workgroup's LDS tiles.
template <int KSEL>
struct Smem {
  // activation tiles and output tiles by tile parity
  __attribute__((aligned(16))) __bf16 xs[2][Cfg<KSEL>::BUF_ELEMS];
  __attribute__((aligned(16))) __bf16 ot_s[2][kTile * kOtRow];
  // target-side (cos, sin) blocks of a tile (tile-blocked table layout) for
  // the epilogue, by tile index mod 3 (keys only)
  __attribute__((aligned(16))) float2 ct_s[3][kTile * kHalf];
};

// One work item: target layer l, head h, keys (KEYS) or values, tokens of
// chunk `chunk`.  Values have no rotation on either side, so their items
// issue no table loads or copies at all.  PAGED: source and target rows
// come from the per-token slot maps (a.src_row, a.dst_row; -1 = skip);
// otherwise row = token.
template <int KSEL, bool PAGED, bool KEYS>
__device__ __forceinline__ void transfer_item(const XferArgs& a, int32_t l, int32_t h, int32_t chunk,
                                              int32_t chunk_tokens, Smem<KSEL>& sm) {
  using C = Cfg<KSEL>;
  constexpr int D = kDepth;
  constexpr bool keys = KEYS;
  // contiguous caches: the matrix waves store the output tiles; paged: the
  // data waves do (they hold the target slot maps)
  constexpr bool kMatrixStores = !PAGED;
  auto& xs = sm.xs;
  auto& ot_s = sm.ot_s;
  auto& ct_s = sm.ct_s;

  const int tid = threadIdx.x;
  // role (0 = matrix waves, 1 = data waves) and wave within the role are
  // wave-uniform; wave q of each role runs on SIMD q
  const int role = __builtin_amdgcn_readfirstlane(tid >> 8);
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
  const int32_t n_tok = (int32_t)a.n_tok;
  const uint32_t src_tok_b = (uint32_t)a.src_tok * 2, dst_tok_b = (uint32_t)a.dst_tok * 2;
  const uint32_t src_bytes = (uint32_t)((a.src_rows - 1) * a.src_tok * 2 + kRowBytes);
  const uint32_t dst_bytes = (uint32_t)((a.dst_rows - 1) * a.dst_tok * 2 + kRowBytes);
  const uint32_t tab_bytes = (uint32_t)((a.n_tok + kTile - 1) / kTile * kCsTileBytes);
  const u32x4 tab_tgt = rsrc_words(a.rope_tgt, tab_bytes);
  {
    const int32_t t_begin = chunk * chunk_tokens;   // a multiple of kTile
    const int32_t t_end = min(t_begin + chunk_tokens, n_tok);
    const int nt = (t_end - t_begin + kTile - 1) / kTile;
    const int32_t blk0 = t_begin / kTile;  // table block of the item's first tile

    // the selected source layers; an out-of-range entry skips the item (the
    // target layer is left unwritten)
    bool active = true;
    rsrc_t srs[KSEL];
#pragma unroll
    for (int j = 0; j < KSEL; ++j) {
      const int32_t sj = a.layer_sel[l * KSEL + j];
      const bool ok = sj >= 0 && sj < a.L_s;
      active = active && ok;
      srs[j] = make_rsrc((const uint16_t*)(keys ? a.src_k : a.src_v) +
                             (ok ? (int64_t)sj * a.src_layer + (int64_t)h * a.src_head : 0),
                         src_bytes);
    }
    if (!active) return;                   // uniform over the workgroup
    const rsrc_t cs_rs = make_rsrc(a.rope_src, tab_bytes);   // source-side tables (keys)
    const int32_t grp = l * a.H + h;
    const uint16_t* W = (const uint16_t*)(keys ? a.W_k : a.W_v) + (int64_t)grp * C::KD * kD;
    const float* bias = (keys ? a.b_k : a.b_v) + (int64_t)grp * kD;
    const rsrc_t dst = make_rsrc((const uint16_t*)(keys ? a.out_k : a.out_v) + (int64_t)l * a.dst_layer +
                                     (int64_t)h * a.dst_head,
                                 dst_bytes);

    bf16x8 wf[C::KSTEPS];       // matrix waves: W^T fragments (see below)
    bf16x8 wb = {}, ones = {};  // matrix waves: the bias step

    // ---- data-wave pieces
    // Issues the loads of tile `tile`'s source rows (this thread's token pt,
    // chunks pc and pc+8 of each selected layer).  Tokens outside the item
    // load zeros.
    auto raw_offset = [&](int tile, Raw<KSEL>& r) __attribute__((always_inline)) {
      const int32_t n = t_begin + tile * kTile + pt;
      const bool ok = tile < nt && n < t_end;
      uint32_t rowb;
      if constexpr (PAGED) {
        rowb = ok && r.row >= 0 ? (uint32_t)r.row * src_tok_b : kSkipRow;
        // slot of this thread's token of the next tile this register set loads
        r.row = a.src_row[max(min(n + D * kTile, t_end - 1), 0)];
      } else {
        rowb = ok ? (uint32_t)n * src_tok_b : kSkipRow;
      }
      return rowb + 16 * pc;
    };
    auto load_layer = [&](Raw<KSEL>& r, uint32_t off, int j) __attribute__((always_inline)) {
      r.lo[j] = __builtin_amdgcn_raw_buffer_load_b128(srs[j], off, 0, 0);
      r.hi[j] = __builtin_amdgcn_raw_buffer_load_b128(srs[j], off + kHalf * 2, 0, 0);
    };
    // tile-blocked table: piece e of (token pt, chunk pc) at e*4KB + pt*128 + pc*16
    auto load_tables = [&](Raw<KSEL>& r, int tile) __attribute__((always_inline)) {
      if constexpr (KEYS) {
        const uint32_t toff = tile < nt ? (uint32_t)(blk0 + tile) * kCsTileBytes + 128 * pt + 16 * pc : kSkipRow;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r.cs[e] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cs_rs, toff + e * (kCsTileBytes / 4), 0, 0));
      }
    };
    auto load_raw = [&](int tile, Raw<KSEL>& r) __attribute__((always_inline)) {
      const uint32_t off = raw_offset(tile, r);
#pragma unroll
      for (int j = 0; j < KSEL; ++j) load_layer(r, off, j);
      load_tables(r, tile);
    };
    // Un-rotates (keys) the register set's rows and writes them into an
    // activation tile (when `use`), refilling the set with tile `next` layer
    // by layer, so that the loads leave between the arithmetic instead of in
    // one burst.  A skipped token's row is zero in, and whatever it becomes
    // only reaches its own output column, which is never stored.
    auto turn_tile = [&](Raw<KSEL>& r, bool use, __bf16* xt, int next) __attribute__((always_inline)) {
      const uint32_t off = raw_offset(next, r);
#pragma unroll
      for (int j = 0; j < KSEL; ++j) {
        if (use) {
          u32x4 lo = r.lo[j], hi = r.hi[j];
          if (keys) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const f32x4 v = r.cs[e];    // (cos, sin) of dims 8pc+2e and 8pc+2e+1
              const float l0 = bf16lo(lo[e]), l1 = bf16hi(lo[e]);
              const float h0 = bf16lo(hi[e]), h1 = bf16hi(hi[e]);
              // R(-p): (lo, hi) -> (lo c + hi s, hi c - lo s)
              lo[e] = pack_bf16(fmaf(l0, v.x, h0 * v.y), fmaf(l1, v.z, h1 * v.w));
              hi[e] = pack_bf16(fmaf(h0, v.x, -(l0 * v.y)), fmaf(h1, v.z, -(l1 * v.w)));
            }
          }
          *(u32x4*)&xt[lds_off<KSEL>(pt, 16 * j + pc)] = lo;
          *(u32x4*)&xt[lds_off<KSEL>(pt, 16 * j + 8 + pc)] = hi;
        }
        load_layer(r, off, j);
        __builtin_amdgcn_sched_barrier(0);
      }
      load_tables(r, next);
    };
    // Writes a computed tile from an LDS output tile to the target cache: 16
    // threads per token row, 16 bytes each, so a wave stores whole 256-byte
    // rows.  read_out fetches this thread's two 16-byte pieces from LDS;
    // write_out issues exactly two stores (a negative tile stores nothing).
    auto read_out = [&](const __bf16* ot, u32x4* v) __attribute__((always_inline)) {
      const int seg = gtid & 15;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) v[hh] = *(const u32x4*)&ot[((gtid >> 4) + 16 * hh) * kOtRow + 8 * seg];
    };
    auto write_out = [&](int tile, const u32x4* v, const int32_t* drow) __attribute__((always_inline)) {
      const int seg = gtid & 15;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = (gtid >> 4) + 16 * hh;
        const int32_t n = t_begin + tile * kTile + r;
        const int32_t row = PAGED ? drow[hh] : n;
        const uint32_t rowb = tile >= 0 && n < t_end && row >= 0 ? (uint32_t)row * dst_tok_b : kSkipRow;
        // non-temporal: the kernel never reads its output back
        __builtin_amdgcn_raw_buffer_store_b128(v[hh], dst, rowb + 16 * seg, 0, kStoreNT);
      }
    };
    // ---- matrix-wave pieces
    // One of the four 1 KB pieces that this wave copies of a tile's (cos,
    // sin) block (keys only): piece q of wave wq is bytes [(4q + wq) KB, +1 KB).
    auto table_piece = [&](const u32x4& table, float2* dst_tab, int tile, int q) __attribute__((always_inline)) {
      if (keys && tile < nt) {
        const uint32_t off = (4 * q + wq) * 1024;
        dma16(table, (uint32_t)(blk0 + tile) * kCsTileBytes + off, (char*)dst_tab + off, 16 * lane);
      }
    };
    // Forward rotation of one finished accumulator block into the LDS
    // output tile ot: half g of this lane's columns.  Accumulator j < 8 is
    // column wcol + 8*(j/4) + 4*lk + j%4 of token lr; j + 8 is its partner
    // 64 columns up.  ec holds the (cos, sin) pieces of those columns.
    auto epilogue_half = [&](const f32x16& acc, const float4* ec, __bf16* ot, int g) __attribute__((always_inline)) {
      const int c0 = wcol + 8 * g + 4 * lk;
      float y0[4] = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      float y1[4] = {acc[8 + 4 * g], acc[9 + 4 * g], acc[10 + 4 * g], acc[11 + 4 * g]};
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
    };
    // The (cos, sin) pieces of this lane's epilogue columns: pieces e = 2lk
    // and 2lk+1 of chunks 2wq and 2wq+1, token lr (tile-blocked layout).
    auto epilogue_tables = [&](const float2* ct_tab, float4* ec) __attribute__((always_inline)) {
      if (keys) {
        const char* tb = (const char*)ct_tab + ep_off;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          ec[2 * g] = *(const float4*)(tb + 16 * g);
          ec[2 * g + 1] = *(const float4*)(tb + 16 * g + kCsTileBytes / 4);
        }
      }
    };
    // One matrix-wave phase: the products Y^T = W^T X^T + b of tile `tile`
    // from xt into acc, with the epilogue of the previous tile (accp, target
    // tables ct_prev, output tile ot_prev) and the copy of the target
    // tables of tile+1 (into ct_next) interleaved between the products, whose
    // dependent chain leaves the wave idle between issues.  The wave ends
    // with the copy of the previous phase complete; this phase's copy stays
    // in flight until the end of the next one.
    auto compute_tile = [&](int tile, const __bf16* xt, f32x16& acc, const f32x16& accp, const float2* ct_prev,
                            __bf16* ot_prev, float2* ct_next, const __bf16* ot_store) __attribute__((always_inline)) {
      // LDS fragments read ahead (with k >= 3 the registers go to W)
      constexpr int kAhead = C::KSTEPS < 8 ? C::KSTEPS : (KSEL >= 3 ? 4 : 8);
      static_assert(8 <= C::KSTEPS, "every table copy and epilogue piece is issued inside the products");
      bf16x8 xf[kAhead];
      float4 ec[4];
      u32x4 ov[2];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) xf[s] = *(const bf16x8*)&xt[lds_off<KSEL>(lr, 2 * s + lk)];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb, ones, f32x16{}, 0, 0, 0);
      epilogue_tables(ct_prev, ec);
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], xf[s % kAhead], acc, 0, 0, 0);
        if (s + kAhead < C::KSTEPS) xf[s % kAhead] = *(const bf16x8*)&xt[lds_off<KSEL>(lr, 2 * (s + kAhead) + lk)];
        if (s < 4) table_piece(tab_tgt, ct_next, tile + 1, s);
        if (s == 4) epilogue_half(accp, ec, ot_prev, 0);
        if (s == 6) epilogue_half(accp, ec, ot_prev, 1);
        if constexpr (kMatrixStores) {
          if (s == 1) read_out(ot_store, ov);
          if (s == C::KSTEPS - 1) write_out(tile - 2, ov, nullptr);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // The matrix waves' only other global accesses are their stores (two
      // per phase, after the copies): the previous phase's four copies are
      // complete once at most its stores and this phase's copies and stores
      // remain.  (Values copy nothing and never wait.)
      if constexpr (KEYS) wait_vmcnt<kMatrixStores ? 8 : 4>();
    };

    // ---- the tile pipeline.  Phase i (i = 0 .. nt+1): the matrix waves
    // compute tile i from xs[i%2] (accumulators kept in registers) while
    // rotating tile i-1 into ot_s[(i-1)%2] with the target tables in
    // ct_s[(i-1)%3], and copy the target tables of tile i+1 into
    // ct_s[(i+1)%3]; the data waves store tile i-2 from ot_s[i%2], un-rotate
    // tile i+1 into xs[(i+1)%2] and issue the loads of tile i+1+D (source
    // rows and source-side tables) into the register set that tile i+1 used
    // (D sets, so loads have D-1 phases to land).  A barrier ends every
    // phase.  The phase loop is unrolled by 6 so that buffer indices and
    // register sets are fixed per copy; the roles run separate loops that
    // meet the same barriers.
    static_assert(6 % D == 0, "register sets cycle with the 6-fold unrolled phase loop");
    lds_barrier();                                   // the previous item's readers of xs[0] are done
    if (role == 0) {
      // W^T fragments of this wave's 32 columns, in registers: lane holds
      // W[m = 16s + 8*lk + i][my_col], i < 8.  The matrix waves stage W
      // through xs[0] 64 rows at a time, transposed on the way in
      // (coalesced 16-byte global loads, 2-byte LDS stores), so that each
      // fragment is one 16-byte LDS read.  (Set up inside the role branch
      // so that the fragments are live only where they are used.)
      __bf16* stage = xs[0];
#pragma unroll
      for (int part = 0; part < C::KD / kStageRows; ++part) {
        const u32x4* gsrc = (const u32x4*)(W + (int64_t)part * kStageRows * kD);
#pragma unroll
        for (int e = gtid; e < kStageRows * kD / 8; e += kGroupThreads) {
          const u32x4 v = gsrc[e];
          const int m = e >> 4, n0 = (e & 15) << 3;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            stage[(n0 + 2 * q) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] & 0xffffu));
            stage[(n0 + 2 * q + 1) * kStageRow + m] = __builtin_bit_cast(__bf16, (uint16_t)(v[q] >> 16));
          }
        }
        lds_barrier();
#pragma unroll
        for (int s4 = 0; s4 < kStageRows / 16; ++s4)
          wf[(kStageRows / 16) * part + s4] = *(const bf16x8*)&stage[my_col * kStageRow + 16 * s4 + 8 * lk];
        lds_barrier();                               // the stage may be overwritten
      }
      // The bias enters the products as one more 16-deep step: A holds the
      // column's fp32 bias split exactly into three bf16 parts (b = b1 + b2
      // + b3), B holds ones in the matching rows, so the accumulator starts
      // at b with no LDS traffic and no epilogue additions.
      if (lk == 0) {
        const float b = bias[my_col];
        const __bf16 b1 = (__bf16)b;
        const __bf16 b2 = (__bf16)(b - (float)b1);
        const __bf16 b3 = (__bf16)(b - (float)b1 - (float)b2);
        wb[0] = b1;
        wb[1] = b2;
        wb[2] = b3;
        ones[0] = ones[1] = ones[2] = (__bf16)1.0f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) table_piece(tab_tgt, ct_s[0], 0, q);
      if constexpr (KEYS) wait_vmcnt<0>();
      lds_barrier();                                 // tile 0 un-rotated
      f32x16 acc[2] = {{}, {}};   // accumulators by tile parity
      auto phase = [&](int i, auto kk) __attribute__((always_inline)) {
        constexpr int K = decltype(kk)::value;      // i % 6
        constexpr int P = K & 1, T = K % 3, Tp = (K + 2) % 3, Tn = (K + 1) % 3;
        if (i < nt) {
          // (in phase 0 the epilogue rotates an empty block into ot_s[1];
          // the data waves never store it)
          compute_tile(i, xs[P], acc[P], acc[P ^ 1], ct_s[Tp], ot_s[P ^ 1], ct_s[Tn], ot_s[P]);
        } else if (i == nt) {
          if constexpr (KEYS) wait_vmcnt<0>();
          float4 ec[4];
          epilogue_tables(ct_s[Tp], ec);
          epilogue_half(acc[P ^ 1], ec, ot_s[P ^ 1], 0);
          epilogue_half(acc[P ^ 1], ec, ot_s[P ^ 1], 1);
        }
        if constexpr (kMatrixStores) {
          if (i >= nt && i <= nt + 1) {   // the last two tiles' stores
            u32x4 ov[2];
            read_out(ot_s[P], ov);
            write_out(i - 2, ov, nullptr);
          }
        }
        (void)T;
        lds_barrier();
      };
      for (int i = 0; i <= nt + 1; i += 6) {
        phase(i, std::integral_constant<int, 0>());
        phase(i + 1, std::integral_constant<int, 1>());
        phase(i + 2, std::integral_constant<int, 2>());
        phase(i + 3, std::integral_constant<int, 3>());
        phase(i + 4, std::integral_constant<int, 4>());
        phase(i + 5, std::integral_constant<int, 5>());
      }
    } else {
      Raw<KSEL> raw[D];
      int32_t drow[2][2] = {{0, 0}, {0, 0}};   // paged: target slots of this thread's rows, by tile parity
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if constexpr (PAGED) raw[d].row = a.src_row[max(min(t_begin + d * kTile + pt, t_end - 1), 0)];
        load_raw(d, raw[d]);
      }
#pragma unroll
      for (int part = 0; part < C::KD / kStageRows; ++part) {   // the matrix waves stage W
        lds_barrier();
        lds_barrier();
      }
      turn_tile(raw[0], true, xs[0], D);
      lds_barrier();                                 // tile 0 un-rotated
      auto phase = [&](int i, auto kk) __attribute__((always_inline)) {
        constexpr int P = decltype(kk)::value & 1;          // i % 2
        constexpr int S = (decltype(kk)::value + 1) % D;    // (i + 1) % D
        // the output reads first: their latency hides behind the un-rotation
        if constexpr (kMatrixStores) {
          turn_tile(raw[S], i + 1 < nt, xs[P ^ 1], i + 1 + D);
        } else {
          u32x4 ov[2];
          read_out(ot_s[P], ov);
          turn_tile(raw[S], i + 1 < nt, xs[P ^ 1], i + 1 + D);
          write_out(i - 2, ov, drow[P]);
        }
        if constexpr (PAGED) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            drow[P ^ 1][hh] = a.dst_row[max(min(t_begin + (i - 1) * kTile + (gtid >> 4) + 16 * hh, t_end - 1), 0)];
        }
        lds_barrier();
      };
      for (int i = 0; i <= nt + 1; i += 6) {
        phase(i, std::integral_constant<int, 0>());
        phase(i + 1, std::integral_constant<int, 1>());
        phase(i + 2, std::integral_constant<int, 2>());
        phase(i + 3, std::integral_constant<int, 3>());
        phase(i + 4, std::integral_constant<int, 4>());
        phase(i + 5, std::integral_constant<int, 5>());
      }
    }
  }
}

// Persistent sweep over the keys (KEYS) or the values of every target
// layer: workgroup b takes items b, b + grid, ...; an item is (token chunk,
// target layer, head) with the head fastest.
template <int KSEL, bool PAGED, bool KEYS>
__global__ void __launch_bounds__(kThreads, 1)
transfer_mfma_kernel(XferArgs a, int32_t n_pairs, int32_t chunk_tokens, int32_t n_items) {
  __shared__ __attribute__((aligned(16))) Smem<KSEL> sm;
  for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int32_t pr = item % n_pairs;
    transfer_item<KSEL, PAGED, KEYS>(a, pr / a.H, pr % a.H, item / n_pairs, chunk_tokens, sm);
  }
}

// CUs of the current device, looked up once per device (safe from any thread)
int cu_count() {
  constexpr int kDevices = 64;
  static std::atomic<int> counts[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
  const int64_t n_pairs = (int64_t)a.L_t * a.H;   // per launch: the keys, then the values
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
#define HELM_LAUNCH(K)                                                                          \
  do {                                                                                          \
    if (paged) {                                                                                \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, true, true>), g, b, 0, stream, a, np, ct, ni);  \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, true, false>), g, b, 0, stream, a, np, ct, ni); \
    } else {                                                                                    \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, false, true>), g, b, 0, stream, a, np, ct, ni); \
      hipLaunchKernelGGL((transfer_mfma_kernel<K, false, false>), g, b, 0, stream, a, np, ct, ni);\
    }                                                                                           \
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
