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
// the matrix cores (40 -> 64 layers, 8 heads, k = 4, IN = 8192, 32,768
// tokens: 70 TFLOP over ~45 GB of compulsory HBM traffic).
//
// Design for MI355X:
//   * Two streaming pre-passes put both operands in k-contiguous bf16, the
//     form the matrix instruction reads: the source keys un-rotated once at
//     src_pos (fp32 arithmetic, rounded once to bf16 — the map's operand
//     type) and each map's W transposed to [D][IN].  Both are HBM-bound and
//     small next to the product (~1 ms of ~72 at the shape above).
//   * Product: v_mfma_f32_32x32x16_bf16, one workgroup per 256-token x
//     256-column tile (two (head, K|V) maps), eight waves of 128 x 64 (two
//     per SIMD, 4 x 2 accumulator blocks, 128 fp32 accumulators per lane).
//     A wave's two 32-column blocks are 64 columns apart in one map, so the
//     RoPE partners d and d+64 sit in the same lane of blocks 0 and 1.  (Four
//     waves of 128 x 128 run at the same speed with twice the registers.)
//   * Operand tiles of 64 k-values reach LDS by buffer->LDS DMA (16 bytes
//     per lane, no registers in between), double-buffered: the copies of
//     step s+1 are issued by four of the eight waves (one per SIMD), one
//     after each of their first 16 products of step s, and land while the
//     rest run.  (The ring
//     depth and step size are parameters; deeper rings of 32-value steps
//     measured slower: one barrier per 32 products instead of 64.)  A lane
//     chooses which 16-byte piece it copies, so the tiles are stored
//     XOR-swizzled (piece c of row r at slot r*8 + (c ^ ((r/2) & 7))) and
//     every 16-byte fragment read of the products is bank-conflict free.
//   * XCD-aware tile order on a persistent grid: the 8 column tiles of a
//     token tile run on one XCD (workgroup id mod 8) at the same time, so
//     its activation tile can be served to all 8 from that XCD's L2.  What bounds it (timed with the copies or the
//     products taken out): the products, LDS reads and barriers alone run at
//     ~59% of the matrix peak; the copies alone move ~9x the compulsory bytes
//     across L2 at ~6 TB/s, because tiles that share operands drift apart in
//     time; together they overlap only partly.  The persistent grid keeps
//     sharers closer than one workgroup per tile did (about 5% faster); a
//     grid-wide lockstep per round of tiles halves the bytes but every tile
//     then waits on the same misses, and neither deeper rings, L2 warm-up
//     loads nor loads staged through registers two steps ahead shortened the
//     wait (vector memory returns in issue order).
//   * Epilogue: bias, the forward rotation at tgt_pos (keys; fp32 tables
//     from the RoPE table kernel) and the rounding to bf16 in registers; the
//     output tile then goes through LDS (the free operand ring), so the
//     stores are whole 256-byte rows, 16 bytes a lane.
#include "internal.hpp"
#include "lds_dma.hpp"

namespace helm {
namespace {

using lds::dma16;
using lds::kSkip;
using lds::lds_barrier;
using lds::rsrc_words;
using lds::wait_vmcnt;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef lds::u32x4 u32x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kMaxRange = 0xffffff00u;   // largest buffer range used (offsets below it never wrap)

// A buffer descriptor from workgroup-uniform values (kept in scalar registers).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* q = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

constexpr int kD = 128;
constexpr int kHalf = 64;
constexpr int kTT = 256;          // tokens per tile
constexpr int kCT = 256;          // output columns per tile (two maps)
constexpr int kKB = 64;           // k-values per pipeline step
constexpr int kBufs = 2;          // LDS ring of operand tiles: copies run kBufs-1 steps ahead
constexpr int kMaxSel = 64;       // selected layers per target layer (the library's limit on k)
constexpr int kWaves = 8;         // 4: 2 x 2 waves of 128 x 128 outputs; 8: 2 x 4 waves of 128 x 64 (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kNB = 16 / kWaves;  // 32-column accumulator blocks per wave
constexpr int kRowPieces = kKB * 2 / 16;   // 16-byte pieces per tile row and step
constexpr int kSwz = 16 / kRowPieces;      // rows sharing one swizzle pattern
constexpr int kRowsPerCopy = 64 / kRowPieces;   // tile rows per 1 KB copy instruction
constexpr int kCopyWaves = 4;     // waves that issue the operand copies: 0..3, one per SIMD
constexpr int kPer = 4 * kRowPieces / kCopyWaves;   // copy instructions per copying wave, operand and step (tile / waves / 1 KB)
constexpr int kMfmaPerStep = (kKB / 16) * 4 * kNB;
constexpr int kCopyStride = kMfmaPerStep / 2 / (2 * kPer) > 0 ? kMfmaPerStep / 2 / (2 * kPer) : 1;   // copies spread over half a step
static_assert(kKB % 16 == 0 && 16 % kRowPieces == 0 && kBufs >= 2 && kBufs <= 5 && (kBufs - 2) * 2 * kPer < 64, "pipeline shape");

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte slot of piece c of tile row r (XOR swizzle, see the header): the
// 16 rows that one pass of a 16-byte LDS read touches land in 16 different
// bank groups.
__device__ __forceinline__ int slot(int r, int c) { return r * kRowPieces + (c ^ ((r / kSwz) % kRowPieces)); }

struct WideArgs {
  const uint16_t* U;          // un-rotated keys [L_s, H, T, D] bf16
  const uint16_t* V;          // values [L_s, H, T, D] bf16
  const uint16_t* WT_k;       // [L_t, H, D, IN] bf16
  const uint16_t* WT_v;
  const float* b_k;           // [L_t, H, D]
  const float* b_v;
  const float2* rope_tgt;     // (cos, sin) at tgt_pos (rope_tgt_index layout)
  const int32_t* layer_sel;   // [L_t, k]
  uint16_t* out_k;            // [L_t, H, T, D] bf16
  uint16_t* out_v;
  int32_t L_s, L_t, H, k, T, IN;
  int32_t n_tt, n_ct;         // token tiles, column tiles per target layer
};

struct GemmSmem {
  uint16_t As[kBufs][kTT * kKB] __attribute__((aligned(16)));
  uint16_t Bs[kBufs][kCT * kKB] __attribute__((aligned(16)));
  int32_t sel[kMaxSel];
};

// One 256 x 256 output tile m, computed by the whole workgroup.
__device__ __forceinline__ void gemm_tile(const WideArgs& a, int64_t m, GemmSmem& sm) {
  auto& As = sm.As;
  auto& Bs = sm.Bs;
  auto& sel_s = sm.sel;

  // ---- tile m: with token tiles a multiple of 8, the column tiles of one
  // token tile are consecutive on one XCD (m mod 8)
  const int64_t per_layer = (int64_t)a.n_tt * a.n_ct;
  const int32_t l = (int32_t)(m / per_layer);
  const int32_t i = (int32_t)(m % per_layer);
  int32_t tt, ct;
  if (a.n_tt % 8 == 0) {
    const int32_t q = i / 8;
    tt = i % 8 + 8 * (q / a.n_ct);
    ct = q % a.n_ct;
  } else {
    tt = i / a.n_ct;
    ct = i % a.n_ct;
  }
  // The selected layers of this target layer, read once into LDS: a global
  // read inside the pipeline would be a vector load, and waiting for it
  // would wait for every copy in flight.  An out-of-range selected layer
  // leaves the target layer unwritten (and no address is ever formed from it).
  if (a.k > kMaxSel) return;
  const int tid = threadIdx.x;
  if (tid < a.k) sel_s[tid] = a.layer_sel[l * a.k + tid];
  __syncthreads();
  for (int j = 0; j < a.k; ++j) {
    const int32_t sj = sel_s[j];
    if (sj < 0 || sj >= a.L_s) return;   // uniform over the workgroup, before any later barrier
  }
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / (kWaves / 2), wn = w % (kWaves / 2);
  // the wave's 32-column blocks: with 8 waves, blocks 32*(wn%2) and +64 of
  // map wn/2, so the RoPE partners d, d+64 sit in one lane of blocks 0 and 1
  auto bcol = [&](int nb) __attribute__((always_inline)) {
    return kWaves == 4 ? 128 * wn + 32 * nb : 128 * (wn >> 1) + 32 * (wn & 1) + 64 * nb;
  };
  const int32_t t0 = tt * kTT;
  const int32_t T = a.T, H = a.H, IN = a.IN;
  const uint32_t slab_bytes = (uint32_t)T * kD * 2;
  const uint32_t map_bytes = (uint32_t)kD * IN * 2;
  const int n_steps = IN / kKB;

  // ---- operand copies: wave w < kCopyWaves issues the A and B copy
  // instructions i = w, w+4, w+8, ... (the other wave of each SIMD issues
  // none, so one wave per SIMD keeps issuing products while its partner
  // waits to issue copies: 58.7-59.1 ms against 59.6-60.2 ms with all eight
  // waves copying; two copying waves ran 65-68 ms); instruction i covers kRowsPerCopy tile rows from
  // kRowsPerCopy*i on, lane q the row kRowsPerCopy*i + q/kRowPieces and slot
  // q % kRowPieces of it (so the piece that swizzles to that slot).  The
  // per-lane byte offsets do not depend on the step; the step's part (which
  // part of a feature block, which k range of W^T) is the uniform scalar
  // offset, and the A descriptor names the step's source slab.  Instruction
  // n of a wave is 4*kRowsPerCopy rows below instruction n-1 and its lanes
  // take the same pieces (the swizzle term repeats every 16*kSwz rows), so
  // one per-lane offset per operand serves all: A adds the row step (and
  // skips rows past T), B folds it, modulo one map, into the scalar offset.
  constexpr int kRowStep = kCopyWaves * kRowsPerCopy;            // rows between a wave's instructions
  constexpr int kMapWraps = kD / kRowStep;                       // instructions per map (B)
  static_assert((16 * kSwz) % kRowStep == 0 || kRowStep % (16 * kSwz) == 0, "swizzle period");
  const int wc = w % kCopyWaves;                                 // (the copying waves' layout)
  const int r0 = kRowsPerCopy * wc + lane / kRowPieces;
  const int c0 = (lane % kRowPieces) ^ ((r0 / kSwz) % kRowPieces);
  const uint32_t voff_a0 = (uint32_t)(t0 + r0) * (kD * 2) + 16 * c0;
  const uint32_t a_lim = (uint32_t)T * (kD * 2);                 // first byte past the last token
  const uint32_t voff_b0 = (uint32_t)r0 * IN * 2 + 16 * c0;
  u32x4 rs_b[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int mi = 2 * ct + q;                            // map: kind * H + head
    rs_b[q] = rsrc_words((mi / H ? a.WT_v : a.WT_k) + ((int64_t)l * H + mi % H) * kD * IN, map_bytes);
  }
  constexpr int kStepsPerBlock = kD / kKB;                // steps per (j, kv, g) feature block
  auto a_rsrc = [&](int s) __attribute__((always_inline)) {
    const int fb = s / kStepsPerBlock;                    // feature block (j, kv, g)
    const int j = fb / (2 * H), kv = (fb / H) & 1, g = fb % H;
    const int32_t sl = __builtin_amdgcn_readfirstlane(sel_s[j]);
    return rsrc_words((kv ? a.V : a.U) + ((int64_t)sl * H + g) * T * kD, slab_bytes);
  };
  // copy q (0 .. 2*kPer-1) of step s into ring slot p: q < kPer this wave's
  // A instruction q, else its B instruction q-kPer (the first half of the B
  // instructions covers map 0, the second map 1)
  auto copy_one = [&](int s, int p, int q, const u32x4& ra) __attribute__((always_inline)) {
    if (w >= kCopyWaves) return;   // wave-uniform
    if (q < kPer) {
      const uint32_t va = voff_a0 + (uint32_t)(q * kRowStep * kD * 2);
      dma16(ra, va < a_lim ? va : kSkip, (uint32_t)(s % kStepsPerBlock) * (kKB * 2),   // (kSkip + 192 stays past every range)
            (const char*)As[p] + 1024 * (wc + kCopyWaves * q));
    } else {
      const int n = q - kPer;
      dma16(rs_b[n >= kPer / 2 ? 1 : 0], voff_b0,
            (uint32_t)s * (kKB * 2) + (uint32_t)((n % kMapWraps) * kRowStep) * (uint32_t)IN * 2,
            (const char*)Bs[p] + 1024 * (wc + kCopyWaves * n));
    }
  };

  f32x16 acc[4][kNB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x16{};

  // steps 0 .. kBufs-2 in flight before the loop (n_steps >= kBufs - 1:
  // at least 256 features, the host checks)
#pragma unroll
  for (int s0 = 0; s0 < kBufs - 1; ++s0) {
    const u32x4 ra = a_rsrc(s0);
#pragma unroll
    for (int q = 0; q < 2 * kPer; ++q) copy_one(s0, s0, q, ra);
  }
  wait_vmcnt<(kBufs - 2) * 2 * kPer>();   // step 0 landed
  lds_barrier();
  // fragment bases: row 128*wm + 32*mb + lane%32 (resp. 128*wn + ...), piece
  // 2*ks + lane/32; the swizzle term depends on lane%32 only, so the four
  // 32-row blocks are 32 rows apart
  const int fr = lane & 31;
  auto frag_off = [&](int base_row, int ks) __attribute__((always_inline)) {
    return slot(base_row + fr, 2 * ks + (lane >> 5)) * 8;
  };
  constexpr int kBlockElems = 32 * kRowPieces * 8;        // one 32-row block of a tile (elements)
  // one pipeline step: the products of step s from ring slot s % kBufs and,
  // with ISSUE, the copies of step s+kBufs-1 into the slot step s-1 used
  auto step = [&](int s, auto issue) __attribute__((always_inline)) {
    constexpr bool kIssue = decltype(issue)::value;
    const int p = s % kBufs;
    const int ahead = s + kBufs - 1;
    u32x4 ra;
    if constexpr (kIssue) ra = a_rsrc(ahead);
    const uint16_t* A = As[p];
    const uint16_t* B = Bs[p];
    bf16x8 af[2][4], bfr[2][kNB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[0][mb] = *(const bf16x8*)&A[frag_off(128 * wm, 0) + mb * kBlockElems];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) bfr[0][nb] = *(const bf16x8*)&B[frag_off(bcol(nb), 0)];
#pragma unroll
    for (int ks = 0; ks < kKB / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kKB / 16) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          af[nxt][mb] = *(const bf16x8*)&A[frag_off(128 * wm, ks + 1) + mb * kBlockElems];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          bfr[nxt][nb] = *(const bf16x8*)&B[frag_off(bcol(nb), ks + 1)];
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mb], bfr[cur][nb], acc[mb][nb], 0, 0, 0);
          // the copies of the step ahead, one after every kCopyStride-th product
          const int m = 4 * kNB * ks + kNB * mb + nb;
          if constexpr (kIssue)
            if (m % kCopyStride == kCopyStride - 1 && m / kCopyStride < 2 * kPer)
              copy_one(ahead, ahead % kBufs, m / kCopyStride, ra);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // steady state: step s+1 must have landed at the end of step s, the copies
  // of steps s+2 .. s+kBufs-1 may still fly
  int s = 0;
  for (; s + kBufs - 1 < n_steps; ++s) {
    step(s, std::true_type{});
    wait_vmcnt<(kBufs - 2) * 2 * kPer>();
    lds_barrier();        // everyone's copies of step s+1 landed; everyone is done with slot s % kBufs
  }
  // the last kBufs-1 steps issue nothing; after step s the copies of steps
  // s+2 .. n_steps-1 (at most two steps' worth) may still fly
  for (; s < n_steps; ++s) {
    step(s, std::false_type{});
    const int rem = n_steps - s - 2;
    if (rem >= 2) wait_vmcnt<2 * 2 * kPer < 64 ? 2 * 2 * kPer : 0>();
    else if (rem == 1) wait_vmcnt<2 * kPer>();
    else wait_vmcnt<0>();
    lds_barrier();
  }

  // ---- epilogue: bias, the forward rotation at tgt_pos (keys), bf16.  The
  // output tile goes through LDS (the operand ring is free once the last
  // step's barrier has passed) so that the stores are whole 256-byte rows,
  // 16 bytes a lane.  LDS tile [map q][token row][16 pieces of 16 bytes],
  // piece j of row r at slot j ^ (r & 15): the two halves of a wave write
  // rows 4 apart, and one row's 16 pieces cover all banks once.
  // Accumulator register r of block (mb, nb) holds row 8*(r/4) + 4*(lane/32)
  // + r%4 of the block, column lane%32.
  static_assert(sizeof(GemmSmem::As) + sizeof(GemmSmem::Bs) >= 2 * kTT * kD * 2 &&
                    offsetof(GemmSmem, Bs) == sizeof(GemmSmem::As),
                "the output tile fits the operand ring (As then Bs)");
  uint16_t* ot = &As[0][0];
  auto ot_at = [](int q, int row, int d) __attribute__((always_inline)) {
    return (q * kTT + row) * kD + 8 * ((d >> 3) ^ (row & 15)) + (d & 7);
  };
  const int q_w = kWaves == 4 ? wn : wn >> 1;             // the wave's map within the tile
  const int mi_w = 2 * ct + q_w;
  const int kind_w = mi_w / H;
  const float* bias = (kind_w ? a.b_v : a.b_k) + ((int64_t)l * H + mi_w % H) * kD;
  const int col = lane & 31, hl = lane >> 5;
  // Key maps: the (cos, sin) of the forward rotation for the lane's 16 rows of
  // a 32-row block are read from the tile's slice of the target table through
  // a buffer descriptor and issued together before the block's arithmetic (a
  // read per element, each waited for before the next, made the epilogue of a
  // key tile tens of microseconds).  In rope_tgt_index's layout the lane's
  // pair i = dlo and rows 8(r/4) + 4 hl + r%4 of a block that starts at a
  // multiple of 32 tokens sit at a per-lane base plus a constant per r.  Rows
  // past the table read zeros; rows past the last token are computed but
  // never stored.
  const int64_t tab_entries = (int64_t)((T + kRopeBlock - 1) / kRopeBlock) * kRopeBlock * kHalf;   // the table's size
  const int64_t tab_left = (tab_entries - (int64_t)t0 * kHalf) * (int64_t)sizeof(float2);
  const rsrc_t tab = make_rsrc(a.rope_tgt + (int64_t)t0 * kHalf, (uint32_t)(tab_left < kMaxRange ? tab_left : kMaxRange));
#pragma unroll
  for (int nb = 0; nb < kNB / 2; ++nb) {
    const int dlo = (kWaves == 4 ? 32 * nb : 32 * (wn & 1)) + col, dhi = dlo + kHalf;
    const float blo = bias[dlo], bhi = bias[dhi];
    const uint32_t lane_tab =
        (uint32_t)((dlo >> 2) * 64 + ((dlo & 3) >> 1) * 32 + 8 * hl + (dlo & 1)) * (uint32_t)sizeof(float2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x2 cs[16];
      if (kind_w == 0) {
        const uint32_t blk = lane_tab + (uint32_t)((128 * wm + 32 * mb) * kHalf * sizeof(float2));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t e = (uint32_t)((r >> 3) * kRopeBlock * kHalf + 16 * ((r >> 2) & 1) + 2 * (r & 3));
          cs[r] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(tab, blk + e * (uint32_t)sizeof(float2), 0, 0));
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
        float ylo = acc[mb][nb][r] + blo, yhi = acc[mb][nb + kNB / 2][r] + bhi;
        if (kind_w == 0) {
          const float olo = fmaf(ylo, cs[r].x, -(yhi * cs[r].y));
          const float ohi = fmaf(yhi, cs[r].x, ylo * cs[r].y);
          ylo = olo;
          yhi = ohi;
        }
        ot[ot_at(q_w, row, dlo)] = __builtin_bit_cast(uint16_t, (__bf16)ylo);
        ot[ot_at(q_w, row, dhi)] = __builtin_bit_cast(uint16_t, (__bf16)yhi);
      }
    }
  }
  lds_barrier();
  // the stores: piece j of row r of map q per thread, 16 threads per row
  for (int g = tid; g < 2 * kTT * 16; g += kThreads) {
    const int q = g / (kTT * 16), row = (g / 16) % kTT, j = g % 16;
    const int32_t t = t0 + row;
    if (t >= T) continue;
    const int mi = 2 * ct + q;
    uint16_t* out = (mi / H ? a.out_v : a.out_k) + (((int64_t)l * H + mi % H) * T + t) * kD;
    *(u32x4*)(out + 8 * j) = *(const u32x4*)&ot[(q * kTT + row) * kD + 8 * (j ^ (row & 15))];
  }
}

// A persistent grid: one workgroup per CU, workgroup b computing tiles b,
// b + grid, b + 2 grid, ...  The sharers of an activation tile (the 8 column
// tiles of a token tile, on one XCD) then start every tile together and,
// doing the same work, stay close enough for the XCD's L2 to serve one
// fetch to all of them; with one workgroup per tile the hardware hands the
// next tile to whichever CU frees first and sharers drift apart.  (Measured
// on the 40 -> 64-layer, 32K-token shape: 61.8-62.7 ms against 64.2-65.6 ms
// for one workgroup per tile.  Rotating each sharer's k-loop start by one or
// more steps, so that one leads and the others follow through L2, ran
// slower: 65.6-66.2 ms.)
__global__ void __launch_bounds__(kThreads, 1) wide_gemm_kernel(WideArgs a) {
  __shared__ GemmSmem sm;
  const int64_t n_tiles = (int64_t)a.L_t * a.n_tt * a.n_ct;
  for (int64_t m = blockIdx.x; m < n_tiles; m += gridDim.x) {
    gemm_tile(a, m, sm);
    __syncthreads();   // the next tile's copies overwrite the output tile in LDS
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
      const float2 c0 = rope_src[rope_src_index(t, 8 * pc + 2 * q, kHalf)];
      const float2 c1 = rope_src[rope_src_index(t, 8 * pc + 2 * q + 1, kHalf)];
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
// grid (IN / 64, D / 64, G).  VEC (W 16-byte aligned): every global access is
// 16 bytes (8 threads a 128-byte row segment), the tile's rows padded to 16-
// byte multiples; otherwise 2-byte accesses.
template <bool VEC>
__global__ void __launch_bounds__(256)
transpose_w_kernel(const uint16_t* __restrict__ W, int32_t IN, uint16_t* __restrict__ WT) {
  const int64_t g = blockIdx.z;
  const int m0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const uint16_t* src = W + g * (int64_t)IN * kD;
  uint16_t* dst = WT + g * (int64_t)kD * IN;
  if constexpr (VEC) {
    constexpr int kP = 72;   // padded row (elements)
    __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kP];
    const int c = threadIdx.x & 7, r = threadIdx.x >> 3;   // piece c of rows r, r + 32
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int rr = r + 32 * k;
      *(u32x4*)&tile[rr * kP + 8 * c] = *(const u32x4*)(src + (int64_t)(m0 + rr) * kD + d0 + 8 * c);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int d = r + 32 * k;   // output row d0 + d: inputs m0 + 8c .. m0 + 8c + 7
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (uint32_t)tile[(8 * c + 2 * j) * kP + d] | ((uint32_t)tile[(8 * c + 2 * j + 1) * kP + d] << 16);
      *(u32x4*)(dst + (int64_t)(d0 + d) * IN + m0 + 8 * c) = v;
    }
  } else {
    __shared__ uint16_t tile[64][66];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) tile[r][tx] = src[(int64_t)(m0 + r) * kD + d0 + tx];
    __syncthreads();
    for (int r = ty; r < 64; r += 4) dst[(int64_t)(d0 + r) * IN + m0 + tx] = tile[tx][r];
  }
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
  return x.D == kD && IN % kKB == 0 && IN / kKB >= kBufs - 1 && (int64_t)x.T * kD * 2 <= 0xffffff00LL && (int64_t)kD * IN * 2 <= 0xffffff00LL &&
         al(x.src_k) && al(x.src_v) && al(x.U) && al(x.WT_k) && al(x.WT_v);
}

hipError_t launch_wide(const WideXfer& x, bool prep, bool product, hipStream_t stream) {
  if (!wide_supports(x)) return hipErrorNotSupported;
  if (x.T <= 0) return hipSuccess;
  const int32_t IN = (int32_t)wide_in_features(x.k, x.H, x.D);
  const int64_t G = (int64_t)x.L_t * x.H;
  if (G > 65535) return hipErrorInvalidValue;
  if (prep) {
    // pre-pass 1: un-rotated keys of every source layer
    const int64_t rows = (int64_t)x.L_s * x.H * x.T;
    hipLaunchKernelGGL(unrotate_keys_kernel, dim3(grid_for(rows * 8)), dim3(256), 0, stream,
                       (const uint16_t*)x.src_k, x.rope_src, rows, x.T, x.U);
    // pre-pass 2: every map's W transposed to [D, IN]
    const dim3 tg(IN / 64, kD / 64, (unsigned)G);
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* Wm = (const uint16_t*)(kv ? x.W_v : x.W_k);
      uint16_t* WTm = kv ? x.WT_v : x.WT_k;
      if ((uintptr_t)Wm % 16 == 0)
        hipLaunchKernelGGL(transpose_w_kernel<true>, tg, dim3(256), 0, stream, Wm, IN, WTm);
      else
        hipLaunchKernelGGL(transpose_w_kernel<false>, tg, dim3(256), 0, stream, Wm, IN, WTm);
    }
  }
  if (!product) return hipGetLastError();
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
  const int64_t n_tiles = (int64_t)x.L_t * a.n_tt * a.n_ct;
  if (n_tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  // one workgroup per CU (a microsecond query next to a ~60 ms launch)
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t grid = n_tiles < cus ? n_tiles : cus;
  hipLaunchKernelGGL(wide_gemm_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace helm
