// transfer_mfma.hip — matrix-core transfer kernel for bf16 storage (gfx950).
//
// What it computes is the whole transfer for two target layers l0, l1 of one
// head h, keys or values, over a range of tokens (pages: "Helm Intelligent
// Routing", section "Why carrying the cache across is the hard part"; the
// Qwen3 cache-mapping write-up, section "A linear bridge, strangely enough,
// suffices"):
//   gather    the k selected source layers' rows of head h and, for keys,
//             un-rotate them at src_pos (R(-p)), rounding the content key
//             once to bf16 — the operand type of the map;
//   product   Y = X W on the matrix cores, bf16 x bf16 -> fp32
//             (v_mfma_f32_16x16x32_bf16), computed as Y^T = W^T X^T;
//   epilogue  + b (the accumulators start at the bias), then for keys the
//             forward rotation R(+p') at tgt_pos — always applied — and a
//             nearest-even store to bf16.
//
// Design for MI355X:
//   * Two target layers per workgroup ("slots").  With 64 target layers x 8
//     heads there are 512 (layer, head) maps per launch; two per workgroup
//     puts all of them on the 256 CUs at once, so every source row is
//     fetched from HBM by one token sweep (one map per workgroup needs two
//     sweeps, reading the selected source layers twice), and the target
//     RoPE tables of a tile serve both slots.  Work items are (token chunk,
//     layer pair, head) with the head fastest: workgroups go to the 8 XCDs
//     round robin, so with 8 heads each XCD maps one head's 64 target layers
//     and its L2 holds that head's source rows for all of them.  Keys and
//     values are two launches; when neither half fills the chip (small
//     shapes) one launch carries both, each map staged once.
//   * One wave per SIMD, each holding W for 64 output columns of one slot
//     (256 registers at k = 4): columns 32c .. 32c+31 and their RoPE
//     partners 64+32c .. 64+32c+31 (c = the wave's half), as four 16-row
//     blocks of Y^T whose rows n and n+64 sit in the same lane and register,
//     so the rotation needs no exchange.  Every 16x16x32 product takes A
//     from registers and B (32 features x 16 tokens) from the LDS
//     activation tile, one read for four products.  The tile is read by two
//     waves per slot instead of four: LDS traffic, not the matrix pipe, is
//     what bounds a design with W for 32 columns per wave.
//   * Every wave also gathers: per 16-token tile, lane (token, 16-byte chunk
//     c, pair lane r) loads chunk c of the low half and its partner chunk of
//     the high half from k of the 2k (slot, layer) source rows, un-rotates
//     them and writes the bf16 result into the tile.  The chunk is the
//     lane's lowest three bits: every eight consecutive lanes read one
//     128-byte line, the pattern the per-CU load path returns fastest (lanes
//     alternating between lines return at about 60% of that rate).  The two
//     lanes of a pair (l, l ^ 8) need the same 8 (cos, sin) pairs; each loads
//     half and they swap the rest by DPP.  The gather's vector-ALU work is
//     interleaved step by step with
//     the product loop of the same wave, so one wave keeps both the matrix
//     pipe and the vector ALU of its SIMD busy.
//   * 16-token tiles, two activation buffers, one LDS barrier per tile.
//     Loads run two tiles ahead (register sets by tile parity), the target
//     tables one tile ahead (shared through LDS), and the output tile is
//     stored from LDS one tile later as whole 256-byte rows, 16 bytes per
//     lane, non-temporal.
//   * No hidden waits.  gfx9 counts outstanding vector memory operations in
//     one in-order counter, so every global access of the tile loop is
//     issued unconditionally (tokens outside the item read a valid row and
//     are never stored; table reads and stores past a range use buffer
//     offsets beyond the descriptor, which read zeros / are dropped): every
//     phase issues the same operations, and the waits the compiler derives
//     are exactly for data that has had its pipeline depth to arrive.
//   * Bias as the products' initial accumulator (exact fp32, no extra work).
//   * W is staged through LDS as stored (32 rows a step, two buffers, the
//     global loads three steps ahead, so that an item pays about one memory
//     latency for its 256 KB of maps: at 512 tokens the staging is most of
//     an item) and turned into A fragments with the transposing
//     ds_read_b64_tr_b16.
#include "internal.hpp"
#include "lds_dma.hpp"

#include <atomic>
#include <type_traits>

namespace helm {
namespace {

using lds::lds_barrier;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kD = 128;          // head dimension
constexpr int kHalf = 64;
constexpr int kThreads = 256;    // 4 waves, one per SIMD
constexpr int kTile = 16;        // tokens per tile = the product's N
constexpr int kRowBytes = kD * 2;
constexpr int kOtRow = kD + 8;   // LDS output row (bf16), 16-byte pad
constexpr int kTabTile = kTile * kHalf;   // float2 entries of one tile's table
constexpr int kStageRows = 32;   // W rows staged per pass (one product step)
constexpr int kStageRow = kD + 8;  // a staged W row (bf16), 16-byte pad
// Byte offset past every descriptor's range: loads there return zero and
// stores are dropped (descriptor ranges stay below it; adding < 256 cannot wrap).
constexpr uint32_t kMaxRange = 0xffffff00u;
constexpr uint32_t kSkip = 0xffffff00u;
constexpr int kStoreNT = 2;      // cache-policy bits of the output stores: nt (streaming)

template <int KSEL>
struct Cfg {
  static constexpr int KD = KSEL * kD;        // product depth
  static constexpr int KSTEPS = KD / 32;      // 16x16x32 steps
  static constexpr int ROW = KD + 8;          // activation row (bf16), 16-byte pad
  static constexpr int NJ = KSEL;             // (slot, layer) rows a gathering lane handles
};

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;   // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// A buffer descriptor from workgroup-uniform values.  The values are passed
// through readfirstlane so that the compiler keeps the descriptor in scalar
// registers (a descriptor it takes for per-lane makes every access a loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* q = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Each lane receives the vector of lane l ^ 8, the other lane of its pair
// (DPP row_ror:8 rotates each row of 16 lanes by half a row).
__device__ __forceinline__ f32x4 pair_swap(const f32x4& v) {
  f32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    o[d] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[d]), 0x128, 0xF, 0xF, false));
  return o;
}

// Activation tile layout.  A token's row holds the k selected layers' 128
// features each; within a layer's 256 bytes, 16-byte chunk c of layer j is
// stored at chunk c ^ X(j), X(j) = 8 (j & 1) + 4 (j >> 1), and the second
// slot's tile starts 128 bytes past a multiple of 256.  The gather writes
// one chunk of two (slot, layer) rows from the two halves of a 16-lane row
// at once; the swizzle and the offset put those halves on different LDS
// banks.  The product reads chunk 4(s%4) + lg of layer s/4 at step s (lg in
// 0..3 is untouched by the XOR), so its element offset is a compile-time
// constant plus 8 lg.
__device__ __forceinline__ constexpr int xswz(int j) { return 8 * (j & 1) + 4 * (j >> 1); }
__device__ __forceinline__ constexpr int kswz(int s) { return kD * (s / 4) + 8 * ((4 * (s % 4)) ^ xswz(s / 4)); }

// What a gathering lane holds of one tile: per (slot, layer) row jj the
// 16-byte chunk of the low half and its partner chunk of the high half, and
// its half of the tile's source (cos, sin) pairs (keys).
template <int KSEL>
struct Raw {
  u32x4 lo[Cfg<KSEL>::NJ], hi[Cfg<KSEL>::NJ];
  f32x4 cs[2];
};

template <int KSEL>
struct Smem {
  static constexpr int SLOT = kTile * Cfg<KSEL>::ROW + 64;   // a slot's tile + 128-byte offset
  union {
    __bf16 act[2][2 * SLOT];                    // [tile parity][slot, token, feature]
    __bf16 stage[2][2][kStageRows * kStageRow]; // W staging: [buffer][slot][row][column]
  };
  __bf16 ot[2][2][kTile * kOtRow];              // [tile parity][slot][token][column]
  float2 ct[3][kTabTile];                       // target (cos, sin) of a tile, by tile index mod 3
  float bias[2][kD];                            // the slots' bias rows
};

// One work item: target layers l0 (slot 0) and l1 (slot 1, none when
// l1 >= L_t), head h, keys (KEYS) or values, tokens [t_begin, t_end).
// PAGED: source and target rows come from the per-token slot maps
// (a.src_row, a.dst_row; -1 = skip); otherwise row = token.
template <int KSEL, bool PAGED, bool KEYS>
__device__ __forceinline__ void transfer_item(const XferArgs& a, int32_t l0, int32_t l1, int32_t h,
                                              int32_t t_begin, int32_t t_end, Smem<KSEL>& sm) {
  using C = Cfg<KSEL>;
  constexpr int NJ = C::NJ;
  constexpr int S = C::KSTEPS;
  constexpr int SLOT = Smem<KSEL>::SLOT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lam = w >> 1, hc = w & 1;                // product role: slot, column half
  const int ln = lane & 15, lg = lane >> 4;          // product lane: token / block row, k-group
  const int gc = lane & 7, gr = (lane >> 3) & 1;     // gathering lane: 16-byte chunk, pair lane
  const int gt = 4 * w + (lane >> 4);                //   and token of the tile
  const int st = tid >> 4, sg = tid & 15;            // storing lane: token, 16-byte segment
  const int nt = (t_end - t_begin + kTile - 1) / kTile;
  const int32_t blk0 = t_begin / kTile;              // table block of the item's first tile

  // ---- the two slots: active when the layer exists and its selection row
  // is in range (an out-of-range entry leaves that target layer unwritten)
  int32_t lay[2] = {l0, l1};
  bool act_slot[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    bool ok = lay[s] < a.L_t;
#pragma unroll
    for (int j = 0; j < KSEL; ++j) {
      const int32_t sj = ok ? a.layer_sel[lay[s] * KSEL + j] : 0;
      ok = ok && sj >= 0 && sj < a.L_s;
    }
    act_slot[s] = ok;
  }
  if (!act_slot[0] && !act_slot[1]) return;          // uniform over the workgroup

  const char* src = (const char*)(KEYS ? a.src_k : a.src_v);
  const uint16_t* Wt = (const uint16_t*)(KEYS ? a.W_k : a.W_v);
  const float* bias = KEYS ? a.b_k : a.b_v;
  const uint32_t src_tok_b = (uint32_t)a.src_tok * 2, dst_tok_b = (uint32_t)a.dst_tok * 2;
  const uint32_t tab_bytes = (uint32_t)((a.n_tok + kTile - 1) / kTile * kTabTile * 8);
  const rsrc_t tab_src = make_rsrc(a.rope_src, tab_bytes);
  const rsrc_t tab_tgt = make_rsrc(a.rope_tgt, tab_bytes);
  // output slots (stores): range 0 when a slot is inactive
  const uint32_t dst_bytes = (uint32_t)((a.dst_rows - 1) * a.dst_tok * 2 + kRowBytes);
  auto dst_of = [&](int s) __attribute__((always_inline)) {
    return make_rsrc((const char*)(KEYS ? a.out_k : a.out_v) +
                         ((int64_t)(act_slot[s] ? lay[s] : 0) * a.dst_layer + (int64_t)h * a.dst_head) * 2,
                     act_slot[s] ? dst_bytes : 0u);
  };
  const rsrc_t dst0 = dst_of(0), dst1 = dst_of(1);

  // ---- gathering lane: base address of each of its (slot, layer) rows
  // (combination c = gr + 2jj: slot c / KSEL, layer c % KSEL; rows of an
  // inactive slot read layer 0: that slot's products are never stored)
  const char* gbase[NJ];
  int gfeat[NJ], gfeat_hi[NJ];
  __bf16* gdst[NJ][2];   // by tile parity
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int c = gr + 2 * jj;
    const int s = c / KSEL, j = c % KSEL;
    const int32_t sl = act_slot[s] ? a.layer_sel[lay[s] * KSEL + j] : 0;
    gfeat[jj] = j * kD + 8 * (gc ^ xswz(j));              // low-half chunk gc, swizzled
    gfeat_hi[jj] = j * kD + 8 * ((gc + 8) ^ xswz(j));     // its partner chunk gc + 8
    gbase[jj] = src + ((int64_t)sl * a.src_layer + (int64_t)h * a.src_head) * 2 + 16 * gc;
#pragma unroll
    for (int p = 0; p < 2; ++p) gdst[jj][p] = sm.act[p] + s * SLOT + gt * C::ROW;
  }
  // Row of the gathering lane's token of tile `tile` (clamped into the item:
  // rows outside it are read but never stored).  Paged caches read the slot
  // maps two phases before their use, ahead of the phase's stores: vector
  // memory operations complete in issue order, so waiting for a map read
  // also waits for every older store, and those are then two phases old.
  auto src_row_of = [&](int tile) __attribute__((always_inline)) -> int32_t {
    const int32_t n = min(t_begin + tile * kTile + gt, t_end - 1);
    if constexpr (PAGED) {
      return a.src_row[n];
    } else {
      return n;
    }
  };
  auto load_row = [&](int32_t row, int jj, Raw<KSEL>& r) __attribute__((always_inline)) {
    const u32x4* p = (const u32x4*)(gbase[jj] + (int64_t)(row >= 0 ? row : 0) * src_tok_b);
    r.lo[jj] = p[0];
    r.hi[jj] = p[kHalf / 8];
  };
  auto load_cs = [&](int tile, Raw<KSEL>& r) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      // pieces e = 2 gr, 2 gr + 1 of (token, chunk): pairs 8c + 2e, 8c + 2e + 1
      const uint32_t off = tile < nt ? (uint32_t)((blk0 + tile) * kTabTile + 2 * gr * 256 + gt * 16 + gc * 2) * 8u
                                     : kSkip;
      r.cs[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tab_src, off, 0, 0));
      r.cs[1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tab_src, off + 256 * 8, 0, 0));
    }
  };
  // One unit of the un-rotation (keys): piece e of row jj, with v = the
  // (cos, sin) of dims 8c+2e and 8c+2e+1.  R(-p): (lo, hi) -> (lo c + hi s,
  // hi c - lo s).
  auto turn_unit = [&](Raw<KSEL>& r, int jj, int e, const f32x4& v) __attribute__((always_inline)) {
    const float l0 = bf16lo(r.lo[jj][e]), l1 = bf16hi(r.lo[jj][e]);
    const float h0 = bf16lo(r.hi[jj][e]), h1 = bf16hi(r.hi[jj][e]);
    r.lo[jj][e] = pack_bf16(fmaf(l0, v.x, h0 * v.y), fmaf(l1, v.z, h1 * v.w));
    r.hi[jj][e] = pack_bf16(fmaf(h0, v.x, -(l0 * v.y)), fmaf(h1, v.z, -(l1 * v.w)));
  };
  // the (cos, sin) of piece e: this lane's (e = 2 gr, 2 gr + 1) or its pair partner's
  auto piece_cs = [&](const Raw<KSEL>& r, int e) __attribute__((always_inline)) {
    const f32x4 own = r.cs[e & 1], other = pair_swap(r.cs[e & 1]);
    return (e >> 1) == gr ? own : other;
  };
  auto put_row = [&](const Raw<KSEL>& r, int jj, int par) __attribute__((always_inline)) {
    *(u32x4*)&gdst[jj][par][gfeat[jj]] = r.lo[jj];
    *(u32x4*)&gdst[jj][par][gfeat_hi[jj]] = r.hi[jj];
  };

  // ---- product lane: W^T fragments of its four blocks (block b: rows
  // 32hc + 16(b%2) + 64(b/2) of Y^T), from LDS staging one step at a time
  bf16x8 wf[S][4];
  {
    const int64_t grp[2] = {(int64_t)(act_slot[0] ? lay[0] : 0) * a.H + h,
                            (int64_t)(act_slot[1] ? lay[1] : 0) * a.H + h};
    // rows 32 s .. 32 s + 31 of both slots' W: 1,024 pieces of 16 bytes,
    // four a thread; loaded three steps ahead, so that the item pays one
    // memory latency instead of one a step
    auto load_step = [&](int s, u32x4* v) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + kThreads * u;
        const int sl = c >> 9, row = (c >> 4) & 31, c16 = c & 15;
        const u32x4* g = (const u32x4*)(Wt + (grp[sl] * C::KD + kStageRows * s + row) * kD + 8 * c16);
        v[u] = act_slot[sl] ? *g : u32x4{0u, 0u, 0u, 0u};
      }
    };
    constexpr int PD = 3;
    u32x4 v[PD][4];
#pragma unroll
    for (int d = 0; d < PD; ++d)
      if (d < S) load_step(d, v[d]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      // staging buffer s % 2 was last read at step s - 2, before the
      // barrier of step s - 1
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + kThreads * u;
        const int sl = c >> 9, row = (c >> 4) & 31, c16 = c & 15;
        *(u32x4*)&sm.stage[s & 1][sl][row * kStageRow + 8 * c16] = v[s % PD][u];
      }
      if (s + PD < S) load_step(s + PD, v[s % PD]);
      lds_barrier();
      // A fragment of block b: lane l gets W[32 s + 8 lg + 0..7][col + ln];
      // within a 16-lane group lane 4e + qq names row (.. + e) and columns
      // 4qq .. 4qq+3, and receives its column of 4 rows
      const int e = ln >> 2, qq = ln & 3;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = 8 * lg + e, col = 32 * hc + 16 * (b & 1) + 64 * (b >> 1) + 4 * qq;
        const __bf16* p = &sm.stage[s & 1][lam][row * kStageRow + col];
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * kStageRow));
        wf[s][b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  }
  // the slots' bias rows into LDS: the accumulators of every tile start at
  // the bias of the lane's rows (columns)
  {
    const int sl = tid >> 7, col = tid & 127;
    sm.bias[sl][col] = act_slot[sl] ? bias[((int64_t)lay[sl] * a.H + h) * kD + col] : 0.f;
  }
  auto load_bias = [&](f32x4* bv) __attribute__((always_inline)) {
    const float* bb = &sm.bias[lam][32 * hc + 4 * lg];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = *(const f32x4*)(bb + 16 * (b & 1) + 64 * (b >> 1));
  };

  // ---- target table: each wave loads four pair groups of the tile's
  // table (groups 4w .. 4w+3, both halves: 2 KB) and puts them into LDS;
  // the epilogue reads its pairs there
  const uint32_t tq_off = (uint32_t)((4 * w + lg) * 64 + ln * 2) * 8u;
  auto load_tq = [&](int tile, f32x4* v) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      const uint32_t off = tile < nt ? (uint32_t)(blk0 + tile) * (kTabTile * 8u) + tq_off : kSkip;
      v[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tab_tgt, off, 0, 0));
      v[1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tab_tgt, off + 32 * 8, 0, 0));
    }
  };
  auto put_tq = [&](const f32x4* v, float2* ct) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      *(f32x4*)((char*)ct + tq_off) = v[0];
      *(f32x4*)((char*)ct + tq_off + 32 * 8) = v[1];
    }
  };

  // ---- epilogue of a finished tile, in two parts per block pair (g = 0:
  // blocks 0, 2; g = 1: blocks 1, 3 — RoPE partners, rows n and n + 64):
  // part hh handles rows 2hh, 2hh + 1 of the lane's four, and the second
  // part writes the four finished columns of both halves into the LDS output
  // tile.  (cos, sin) of pairs 32hc + 16g + 4lg + 0..3 sit in table group
  // 8hc + 4g + lg.
  auto epi_tables = [&](const float2* ct, int g, f32x4* cv) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      const char* tb = (const char*)ct + (uint32_t)((8 * hc + 4 * g + lg) * 64 + ln * 2) * 8u;
      cv[0] = *(const f32x4*)tb;              // pairs 4G, 4G+1
      cv[1] = *(const f32x4*)(tb + 32 * 8);   // pairs 4G+2, 4G+3
    }
  };
  auto epi_part = [&](const f32x4* acc, const f32x4* cv, __bf16* ot, int g, int hh, uint32_t* pk)
                      __attribute__((always_inline)) {
    float y0[2] = {acc[g][2 * hh], acc[g][2 * hh + 1]};
    float y1[2] = {acc[g + 2][2 * hh], acc[g + 2][2 * hh + 1]};
    if constexpr (KEYS) {
      const f32x4 v = cv[hh];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float c = q ? v.z : v.x, sn = q ? v.w : v.y;
        // R(+p'): (lo, hi) -> (lo c - hi s, hi c + lo s)
        const float o0 = fmaf(y0[q], c, -(y1[q] * sn));
        const float o1 = fmaf(y1[q], c, y0[q] * sn);
        y0[q] = o0;
        y1[q] = o1;
      }
    }
    pk[hh] = pack_bf16(y0[0], y0[1]);
    pk[2 + hh] = pack_bf16(y1[0], y1[1]);
    if (hh == 1) {
      const int c0 = 32 * hc + 16 * g + 4 * lg;
      *(uint2*)&ot[ln * kOtRow + c0] = make_uint2(pk[0], pk[1]);
      *(uint2*)&ot[ln * kOtRow + c0 + kHalf] = make_uint2(pk[2], pk[3]);
    }
  };
  // ---- stores of a finished tile: token st, 16-byte segment sg, both slots;
  // `row` is the token's target row (paged: its slot, -1 = skip)
  auto dst_row_of = [&](int tile) __attribute__((always_inline)) -> int32_t {
    const int32_t n = t_begin + tile * kTile + st;
    if constexpr (PAGED) {
      return a.dst_row[max(min(n, t_end - 1), 0)];
    } else {
      return n;
    }
  };
  auto read_out = [&](__bf16 (*ot)[kTile * kOtRow], u32x4* v) __attribute__((always_inline)) {
    v[0] = *(const u32x4*)&ot[0][st * kOtRow + 8 * sg];
    v[1] = *(const u32x4*)&ot[1][st * kOtRow + 8 * sg];
  };
  auto write_out = [&](int tile, int32_t row, const u32x4* v) __attribute__((always_inline)) {
    const int32_t n = t_begin + tile * kTile + st;
    const uint32_t off = tile >= 0 && n < t_end && row >= 0 ? (uint32_t)row * dst_tok_b + 16 * sg : kSkip;
    // non-temporal: the kernel never reads its output back
    __builtin_amdgcn_raw_buffer_store_b128(v[0], dst0, off, 0, kStoreNT);
    __builtin_amdgcn_raw_buffer_store_b128(v[1], dst1, off, 0, kStoreNT);
  };

  // ---- prologue: tile 0 gathered, tile 1 loaded, tile 2 loading, the
  // target table of tile 0 in LDS, the bias of tile 0's accumulators read
  // (paged: the slots of tiles 3 and 4's rows loading)
  lds_barrier();                                     // staging reads done: the tiles may be written
  Raw<KSEL> raw[2];
  f32x4 accs[2][4];
  f32x4 bv[4];
  int32_t srow[2] = {0, 0}, drow[2] = {0, 0};
  {
    f32x4 tq[2];
    load_tq(0, tq);
    const int32_t r0 = src_row_of(0), r1 = src_row_of(1);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) load_row(r0, jj, raw[0]);
    load_cs(0, raw[0]);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) load_row(r1, jj, raw[1]);
    load_cs(1, raw[1]);
    put_tq(tq, sm.ct[0]);
  }
  if constexpr (KEYS) {
#pragma unroll
    for (int u = 0; u < NJ * 4; ++u) turn_unit(raw[0], u % NJ, u / NJ, piece_cs(raw[0], u / NJ));
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) put_row(raw[0], jj, 0);
  {
    const int32_t r2 = src_row_of(2);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) load_row(r2, jj, raw[0]);
    load_cs(2, raw[0]);
  }
  if constexpr (PAGED) {
    srow[0] = src_row_of(3);
    srow[1] = src_row_of(4);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) accs[1][b] = f32x4{0.f, 0.f, 0.f, 0.f};   // "tile -1": never stored
  load_bias(bv);
  lds_barrier();

  // ---- the tile pipeline.  Phase i works on five tiles at once, spread
  // over the product steps of tile i so that the matrix pipe, the vector
  // ALU, LDS and the memory path all stay busy:
  //   products of tile i (activation buffer i % 2, accumulators i % 2),
  //   gather of tile i+1 (loaded in phase i-2) into the other buffer and
  //     the loads of tile i+3 into the register set it frees,
  //   epilogue of tile i-1 (the other accumulators, target table i-1) into
  //     output tile (i-1) % 2,
  //   stores of tile i-2 from output tile i % 2,
  //   the target table of tile i+1 (tables by tile index mod 3).
  // One barrier ends the phase.  Unrolled by two so that every buffer and
  // register set is fixed; past the last tile the work runs on stale
  // buffers whose results are never stored (so the phase has no branches).
  constexpr int kTq = 0;                       // step of each piece of work
  constexpr int kTqPut = S - 1;
  constexpr int kCv0 = S > 1 ? 1 : 0, kCv1 = S > 3 ? 3 : S - 1;
  constexpr int kOt = S > 4 ? 4 : S - 1, kSt = S > 6 ? 6 : S - 1;
  auto epi_step = [](int g, int hh) constexpr { return 2 + 2 * g + hh < S ? 2 + 2 * g + hh : S - 1; };
  auto put_step = [](int jj) constexpr {
    // keys: after the row's last un-rotation unit (units go piece by piece)
    return KEYS ? 3 * NJ + jj : (jj + 1 < S ? jj + 1 : S - 1);
  };
  auto phase = [&](int i, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;   // i % 2
    constexpr int RA = 3;                     // fragment ring: reads RA - 1 steps ahead
    Raw<KSEL>& r = raw[P ^ 1];
    f32x4* acc = accs[P];
    const f32x4* pacc = accs[P ^ 1];
    const __bf16* xb = sm.act[P] + lam * SLOT + ln * C::ROW + 8 * lg;
    __bf16* ot_prev = sm.ot[P ^ 1][lam];
    const float2* ct_prev = sm.ct[(i + 2) % 3];   // tile i-1
    float2* ct_next = sm.ct[(i + 1) % 3];         // tile i+1
    u32x4 so[2];
    f32x4 cv[2][2];
    f32x4 tq[2];
    uint32_t pk[2][4];
    f32x4 v = {};
    const int32_t row3 = PAGED ? srow[P] : src_row_of(i + 3);
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = bv[b];
    bf16x8 xf[RA];
#pragma unroll
    for (int s = 0; s < RA - 1; ++s) xf[s] = *(const bf16x8*)(xb + kswz(s));
#pragma unroll
    for (int s = 0; s < S; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + RA - 1 < S) xf[(s + RA - 1) % RA] = *(const bf16x8*)(xb + kswz(s + RA - 1));
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s][b], xf[s % RA], acc[b], 0, 0, 0);
      if constexpr (KEYS) {
        // unit s: piece e = s / NJ of row jj = s % NJ
        const int e = s / NJ, jj = s % NJ;
        if (jj == 0) v = piece_cs(r, e);
        turn_unit(r, jj, e, v);
      }
      if (s == 0 && PAGED) {
        srow[P] = src_row_of(i + 5);
      }
      if (s == kTq) load_tq(i + 1, tq);
      if (s == kCv0) epi_tables(ct_prev, 0, cv[0]);
      if (s == kCv1) epi_tables(ct_prev, 1, cv[1]);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (s == epi_step(g, hh)) epi_part(pacc, cv[g], ot_prev, g, hh, pk[g]);
      if (s == kOt) read_out(sm.ot[P], so);
      if (s == kSt) write_out(i - 2, PAGED ? drow[P] : dst_row_of(i - 2), so);
      if (s == kSt && PAGED) drow[P] = dst_row_of(i);   // for phase i + 2's stores
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        if (s == put_step(jj)) {
          put_row(r, jj, P ^ 1);
          load_row(row3, jj, r);
          if (jj == NJ - 1) load_cs(i + 3, r);
        }
      if (s == kTqPut) {
        put_tq(tq, ct_next);
        load_bias(bv);                        // for the next phase's accumulators
      }
      // the fragment stays live to the end of the step, so that the vector
      // work of the step does not reuse its registers and can run beside
      // the products
      asm volatile("" ::"v"(xf[s % RA]));
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };
  for (int i = 0; i <= nt + 1; i += 2) {
    phase(i, std::integral_constant<int, 0>());
    phase(i + 1, std::integral_constant<int, 1>());
  }
}

// Persistent sweep: workgroup b takes items b, b + grid, ...; item =
// (chunk * n_lpairs + layer pair) * H + head, the head fastest.
template <int KSEL, bool PAGED, bool KEYS>
__global__ void __launch_bounds__(kThreads, 1)
transfer_mfma_kernel(XferArgs a, int32_t n_lpairs, int32_t chunk_tokens, int32_t n_items) {
  __shared__ __attribute__((aligned(16))) Smem<KSEL> sm;
  for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int32_t h = item % a.H, rest = item / a.H;
    const int32_t lp = rest % n_lpairs, chunk = rest / n_lpairs;
    const int32_t t_begin = chunk * chunk_tokens;
    const int32_t t_end = (int32_t)min((int64_t)t_begin + chunk_tokens, a.n_tok);
    transfer_item<KSEL, PAGED, KEYS>(a, lp, lp + n_lpairs, h, t_begin, t_end, sm);
    lds_barrier();   // the next item's staging overwrites the tiles
  }
}

// Keys and values in one launch, for shapes too small to fill the chip with
// either half: items [0, n_items) map keys, [n_items, 2 n_items) values, each
// decoded as in transfer_mfma_kernel.  Which half a workgroup maps is uniform
// over the workgroup.
template <int KSEL, bool PAGED>
__global__ void __launch_bounds__(kThreads, 1)
transfer_mfma_kv_kernel(XferArgs a, int32_t n_lpairs, int32_t chunk_tokens, int32_t n_items) {
  __shared__ __attribute__((aligned(16))) Smem<KSEL> sm;
  for (int32_t it = blockIdx.x; it < 2 * n_items; it += gridDim.x) {
    const bool keys = it < n_items;
    const int32_t item = keys ? it : it - n_items;
    const int32_t h = item % a.H, rest = item / a.H;
    const int32_t lp = rest % n_lpairs, chunk = rest / n_lpairs;
    const int32_t t_begin = chunk * chunk_tokens;
    const int32_t t_end = (int32_t)min((int64_t)t_begin + chunk_tokens, a.n_tok);
    if (keys)
      transfer_item<KSEL, PAGED, true>(a, lp, lp + n_lpairs, h, t_begin, t_end, sm);
    else
      transfer_item<KSEL, PAGED, false>(a, lp, lp + n_lpairs, h, t_begin, t_end, sm);
    lds_barrier();   // the next item's staging overwrites the tiles
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

// Token chunks per (layer pair, head): as many as keep every CU busy in as
// few rounds as possible, counting a few tiles of pipeline fill and map
// staging per item.
int64_t pick_chunks(int64_t n_tok, int64_t base_items, int64_t slots) {
  int64_t best = 1, best_cost = INT64_MAX;
  for (int64_t c = 1; c <= 64; ++c) {
    const int64_t items = c * base_items;
    const int64_t rounds = (items + slots - 1) / slots;
    const int64_t chunk = ((n_tok + c - 1) / c + kTile - 1) / kTile * kTile;
    if (c > 1 && (c - 1) * chunk >= n_tok) break;   // chunks would be empty
    const int64_t cost = rounds * (chunk / kTile + 4);
    if (cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// Whether one launch of both halves (c1 token chunks each, every item on a
// CU of its own) is expected to finish before the two launches with c2
// chunks.  Cost in sixteen-token tiles of the values launch: a keys tile
// takes about 1.5 of them, and an item about 18 more for its map staging,
// pipeline fill and drain (measured on the 28 -> 28-layer pair at 512 and
// 2,048 tokens).
bool fused_is_cheaper(int64_t n_tok, int64_t base, int64_t slots, int64_t c2, int64_t c1) {
  auto tiles = [&](int64_t c) { return ((n_tok + c - 1) / c + kTile - 1) / kTile; };
  const int64_t rounds2 = (c2 * base + slots - 1) / slots;
  const int64_t two = rounds2 * (3 * tiles(c2) + 36) + rounds2 * (2 * tiles(c2) + 36);   // doubled units
  const int64_t one = 3 * tiles(c1) + 36;
  return one < two;
}

}  // namespace

bool mfma_supports(const XferArgs& a) {
  // 16-byte vector loads of source rows, W and bias, 16-byte stores of
  // outputs, and the buffer descriptors' byte ranges below kMaxRange
  auto al = [](const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; };
  const int64_t lim = kMaxRange;
  const bool ranges = (a.n_tok + kTile - 1) / kTile * kTabTile * 8 <= lim &&
                      (a.dst_rows - 1) * a.dst_tok * 2 + kRowBytes <= lim && a.n_tok < 0x7fffffffLL &&
                      a.src_tok * 2 <= 0xffffffffLL;
  return ranges && a.D == kD && a.k >= 1 && a.k <= 4 && al(a.src_k, 16) && al(a.src_v, 16) && al(a.W_k, 16) &&
         al(a.W_v, 16) && al(a.out_k, 16) && al(a.out_v, 16) && al(a.rope_src, 16) && al(a.rope_tgt, 16) &&
         al(a.b_k, 16) && al(a.b_v, 16) && (a.src_tok * 2) % 16 == 0 && (a.src_head * 2) % 16 == 0 &&
         (a.src_layer * 2) % 16 == 0 && (a.dst_tok * 2) % 16 == 0 && (a.dst_head * 2) % 16 == 0 &&
         (a.dst_layer * 2) % 16 == 0;
}

hipError_t launch_transfer_mfma(const XferArgs& a, hipStream_t stream) {
  if (!mfma_supports(a)) return hipErrorNotSupported;
  if (a.n_tok <= 0) return hipSuccess;
  const int64_t n_lpairs = (a.L_t + 1) / 2;
  const int64_t base = n_lpairs * a.H;
  const int64_t slots = cu_count();   // one 4-wave workgroup per CU
  const int64_t n_chunks = pick_chunks(a.n_tok, base, slots);
  const int64_t chunk_tokens = ((a.n_tok + n_chunks - 1) / n_chunks + kTile - 1) / kTile * kTile;
  const int64_t chunks = (a.n_tok + chunk_tokens - 1) / chunk_tokens;
  const int64_t n_items = base * chunks;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t grid = n_items < slots ? n_items : slots;
  const dim3 g((unsigned)grid), b(kThreads);
  const int32_t np = (int32_t)n_lpairs, ct = (int32_t)chunk_tokens, ni = (int32_t)n_items;
  const bool paged = a.src_row != nullptr;
  if (paged != (a.dst_row != nullptr)) return hipErrorInvalidValue;
  // both halves in one launch when neither fills the chip and that is cheaper
  const int64_t c1 = slots / (2 * base);
  if (c1 >= 1 && fused_is_cheaper(a.n_tok, base, slots, n_chunks, c1)) {
    const int64_t ct1 = ((a.n_tok + c1 - 1) / c1 + kTile - 1) / kTile * kTile;
    const int64_t items1 = base * ((a.n_tok + ct1 - 1) / ct1);   // <= slots / 2
    const dim3 g1((unsigned)(2 * items1)), b1(kThreads);
    const int32_t ct1i = (int32_t)ct1, ni1 = (int32_t)items1;
#define HELM_LAUNCH_KV(K)                                                                         \
  do {                                                                                            \
    if (paged)                                                                                    \
      hipLaunchKernelGGL((transfer_mfma_kv_kernel<K, true>), g1, b1, 0, stream, a, np, ct1i, ni1);  \
    else                                                                                          \
      hipLaunchKernelGGL((transfer_mfma_kv_kernel<K, false>), g1, b1, 0, stream, a, np, ct1i, ni1); \
  } while (0)
    switch (a.k) {
      case 1: HELM_LAUNCH_KV(1); break;
      case 2: HELM_LAUNCH_KV(2); break;
      case 3: HELM_LAUNCH_KV(3); break;
      default: HELM_LAUNCH_KV(4); break;
    }
#undef HELM_LAUNCH_KV
    return hipGetLastError();
  }
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
