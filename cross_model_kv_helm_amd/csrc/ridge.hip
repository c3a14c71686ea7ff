// ridge.hip — the ridge fit of the maps (the Qwen3 cache-mapping write-up,
// section "A linear bridge, strangely enough, suffices": every target head's
// key map and value map are fitted separately, by ridge regression on
// centred data with lambda = 0.01, the bias from the means).
//
// Per group g (one (target layer, head, K|V) map) with observations
// X [N, IN] and targets Y [N, D]:
//   W = (Xc^T Xc + lambda I)^-1 Xc^T Yc,   b = mean(Y) - mean(X) W
// (Xc, Yc the centred data).  The centred products follow from one pass
// over shifted data D = X - 1 s^T, E = Y - 1 t^T (per-feature shifts s,
// t): Xc^T Xc = D^T D - sd sd^T / N and Xc^T Yc = D^T E - sd se^T / N with
// the column sums sd, se of the shifted data, and mean(X) = s + sd / N.
// Centring is what keeps the fp32 sums accurate: with a feature mean m
// large against its spread sigma, the raw products' partial sums grow like
// n m^2 and their rounding, left in the centred result, like u n m^2 —
// a relative error of order u (m / sigma)^2.  The shifts bring the fed
// values to the order of sigma before any product.  They are taken from the
// group's first observations (ridge_shift_kernel): a feature whose first
// min(N, 64) values share one sign and lie within a factor 1.5 of each
// other is shifted by its first value, any other by 0.  For a shifted
// feature every value within a factor 2 of the shift differs from it by a
// bf16 number exactly (the products stay exact); a rarer value is rounded
// to bf16 once, an error far below the fp32 accumulation's.
//
// Design for MI355X:
//   * Gram kernel (matrix cores, the hot loop: 2 N IN (IN + D) flop per
//     group): X^T X and X^T Y contract over the observations, but X is
//     stored observation-major, so a fragment (8 observations of one
//     feature per lane) is not contiguous in memory.  Operand tiles of 64
//     observations x 256 features are copied to LDS as they are stored
//     (buffer -> LDS DMA, double-buffered) and every fragment is read with
//     two ds_read_b64_tr_b16.  Within each 16-lane group, lane 4e+q gives
//     the address of 4 consecutive features (4q .. 4q+3) of observation e,
//     and lane i receives element i%4 of the 4-feature chunks named by lanes
//     i/4, 4+i/4, 8+i/4, 12+i/4 (a measured lane layout): feature i of
//     observations 0..3, the transpose a fragment needs.  Tile rows
//     are XOR-swizzled in 16-byte pieces (slot = piece ^ 4*((t%4) + 4*((t/8)%2)))
//     so the 8 observation rows one read touches fall in 8 different bank
//     groups.  A wave owns a 128 x 128 block (fp32 accumulators); a
//     workgroup's four waves share its two operand tiles, and one group's
//     workgroups run on one XCD.  Only the blocks on and above the diagonal
//     of the symmetric X^T X are formed.  A diagonal tile (X feature groups
//     2r, 2r+1) needs one operand tile for its three blocks, so its second
//     tile holds Y and its fourth wave forms the X^T Y block of group 2r; the
//     X^T Y blocks of the odd groups go two to a workgroup as 128 x 64
//     halves.  At IN = 512 that is 4 workgroups per group with every wave
//     busy.  The waves of the diagonal blocks read one fragment set for both
//     operands and form the column sums from it with v_dot2_f32_bf16 against
//     ones (vector ALU that the products leave idle), as does the wave that
//     holds Y's fragments.
//   * Solve kernel (fp64, one workgroup per group): the centred normal
//     matrix plus lambda I in upper storage, a blocked Cholesky A = U^T U in
//     16-wide panels with the forward substitution of the right-hand sides
//     folded into the panel updates, then the back substitution, W in fp32
//     and b from the means.  Each panel pass reads and writes the trailing
//     part of the group's fp64 matrix (2.6 MB at IN = 512, beyond L2 and the
//     last-level cache for 1,024 groups), so the kernel is bound by those
//     HBM passes; each memory loop issues 8 rows' accesses at once (32 in
//     the setup pass), the back substitution stages its column block of U
//     in LDS, and the panel rows sit in LDS sized to IN.  At IN <= 512 two
//     workgroups share a CU (80 KB of LDS each), so two groups' memory
//     latency overlaps.
#include "internal.hpp"
#include "lds_dma.hpp"

#include <type_traits>

namespace helm {
namespace {

using lds::dma16;
using lds::kSkip;
using lds::lds_barrier;
using lds::rsrc_words;
using lds::wait_vmcnt;
typedef lds::u32x4 u32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 128;            // target features per map
constexpr int kFT = 256;           // features per tile side
constexpr int kKB = 64;            // observations per pipeline step
constexpr int kRowBytes = kFT * 2; // one observation row of a tile (512 B, 32 pieces)
constexpr int kThreads = 256;
constexpr int kPer = 8;            // copy instructions per wave, operand and step (32 KB tile / 4 waves / 1 KB)
constexpr int kMaxIn = 1024;       // largest input width the solve kernel holds

constexpr int kGroupW = 128;       // features per group: one wave's block side
constexpr int kYTile = -2;         // a B tile that holds Y (pieces 0-15) instead of X groups

struct GramArgs {
  const uint16_t* X;     // [G, N, IN] bf16
  const uint16_t* Y;     // [G, N, D] bf16
  float* shift;          // [G, IN + D] fp32: the shifts of X's features, then of Y's columns
  float* gram;           // [G, IN, IN] fp32 (the 128-blocks on and above the diagonal written)
  float* cross;          // [G, IN, D] fp32
  float* sums;           // [G, IN + D] fp32: column sums of the shifted X, then of the shifted Y
  int64_t N;
  int32_t G, IN, nF;     // nF = IN / 128 feature groups
  int32_t tiles;         // workgroups per group (ridge_tiles_per_group)
};

// The operand tiles of a workgroup: which 128-feature groups of X its A
// tile holds in pieces 0-15 and 16-31 (-1: none, read as zeros), and the
// same for its B tile, or b0 = kYTile: the B tile holds Y.
struct TileJob {
  int a0, a1, b0, b1;
};

// What one wave computes (wave-uniform).
enum Mode {
  kIdle = 0,     // copies only
  kFull = 1,     // a 128 x 128 block
  kFullSumA = 2, // a diagonal 128 x 128 block (B = A) and the column sums of its features
  kFullSumB = 3, // a 128 x 128 block of X^T Y and the column sums of Y
  kHalfY = 4     // a 128 x 64 block of X^T Y
};
struct WaveJob {
  int mode;
  int a_p0, b_p0;   // first 16-byte piece of the wave's A rows / B columns in its tile
  bool b_in_a;      // B columns come from the A tile
  bool cross;       // the block belongs to X^T Y (else X^T X)
  int row0, col0;   // the block's first row (feature) and column (feature or Y column)
  int sum0;         // first sums entry the wave writes (kFullSumA / kFullSumB)
};

// The work of workgroup (tile) t of a group: first the diagonal tiles r <
// nD = ceil(nF/2) (groups 2r, 2r+1: their three X^T X blocks on three
// waves, the X^T Y block of group 2r on the fourth, with Y in the B tile
// that a diagonal tile does not otherwise need), then the off-diagonal
// tiles (r, c), r < c, in row order (four X^T X blocks), then the X^T Y
// blocks of the odd groups two per tile, as 128 x 64 halves on four waves.
// The column sums ride on the waves that already hold the fragments: the
// diagonal blocks' waves sum their features, the first tile's X^T Y wave
// sums Y.
__device__ __forceinline__ void decode_tile(const GramArgs& a, int t, int w, TileJob& tj, WaveJob& wj) {
  const int nF = a.nF, nD = (nF + 1) / 2, nP = nD * (nD - 1) / 2;
  const int wm = w >> 1, wn = w & 1;
  auto grp = [&](int i) { return i < nF ? i : -1; };
  wj = WaveJob{kIdle, 0, 0, false, false, 0, 0, 0};
  if (t < nD) {
    const int r = t, f0 = kGroupW * 2 * r, f1 = f0 + kGroupW;
    tj = TileJob{2 * r, grp(2 * r + 1), kYTile, -1};
    const bool two = tj.a1 >= 0;
    if (w == 0)
      wj = WaveJob{kFullSumA, 0, 0, true, false, f0, f0, f0};
    else if (w == 1 && two)
      wj = WaveJob{kFull, 0, 16, true, false, f0, f1, 0};
    else if (w == 2)
      wj = WaveJob{r == 0 ? kFullSumB : kFull, 0, 0, false, true, f0, 0, a.IN};
    else if (w == 3 && two)
      wj = WaveJob{kFullSumA, 16, 16, true, false, f1, f1, f1};
  } else if (t < nD + nP) {
    int left = t - nD, r = 0;
    while (left >= nD - 1 - r) {
      left -= nD - 1 - r;
      ++r;
    }
    const int c = r + 1 + left;
    tj = TileJob{2 * r, grp(2 * r + 1), 2 * c, grp(2 * c + 1)};
    const int ga = wm ? tj.a1 : tj.a0, gb = wn ? tj.b1 : tj.b0;
    if (ga >= 0 && gb >= 0) wj = WaveJob{kFull, 16 * wm, 16 * wn, false, false, kGroupW * ga, kGroupW * gb, 0};
  } else {
    const int ci = t - nD - nP;
    tj = TileJob{4 * ci + 1, grp(4 * ci + 3), kYTile, -1};
    const int ga = wm ? tj.a1 : tj.a0;
    if (ga >= 0) wj = WaveJob{kHalfY, 16 * wm, 8 * wn, false, true, kGroupW * ga, 64 * wn, 0};
  }
}

// Swizzle of observation row t (multiples of 4 in 0..28: XOR on piece bits 2..4).
__device__ __forceinline__ int row_swz(int t) { return 4 * ((t & 3) + 4 * ((t >> 3) & 1)); }

__device__ __forceinline__ bf16x8 read_frag(const char* tile, uint32_t lane_off, int ks) {
  // rows 16ks + 4r + (lane's e and k-group): the uniform part of the address
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + lane_off + (16 * ks) * kRowBytes));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + lane_off + (16 * ks + 4) * kRowBytes));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// s + the sum of the 8 values of a fragment (v_dot2_f32_bf16 against ones)
__device__ __forceinline__ float frag_sum(const bf16x8& v, float s) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, s, false);
}

// x - s for the 8 values of a fragment (ns = -s): each difference formed
// exactly in fp32 (v_dot2_f32_bf16 against the selectors e0 = (1, 0) and
// e1 = (0, 1), accumulator -s), then rounded to bf16.  Fragment value j is
// observation 8 kg + j of its 16-observation slice; with `n_valid` < 16
// (the group's last slice) the values of later observations (padding read
// as zeros) become 0.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 shift_frag(const bf16x8& v, float ns, int first, int n_valid, bf16x2 e0,
                                             bf16x2 e1) {
  bf16x8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 pr = {v[2 * k], v[2 * k + 1]};
    float d0 = __builtin_amdgcn_fdot2_f32_bf16(pr, e0, ns, false);
    float d1 = __builtin_amdgcn_fdot2_f32_bf16(pr, e1, ns, false);
    if (n_valid < 16) {
      d0 = first + 2 * k < n_valid ? d0 : 0.f;
      d1 = first + 2 * k + 1 < n_valid ? d1 : 0.f;
    }
    o[2 * k] = (__bf16)d0;
    o[2 * k + 1] = (__bf16)d1;
  }
  return o;
}

struct GramSmem {
  char A[2][kKB * kRowBytes] __attribute__((aligned(16)));
  char B[2][kKB * kRowBytes] __attribute__((aligned(16)));
};

// SHIFT: the wave's fragments are shifted (ns_a, ns_b: minus the shifts of
// its A rows' and B columns' features, per 32-block); otherwise every shift
// of the wave is 0 and the fragments are fed as stored.
template <int MODE, bool SHIFT>
__device__ __forceinline__ void gram_steps(const GramArgs& a, GramSmem& sm, int64_t g, const TileJob& tj,
                                           const WaveJob& wj, int w, int lane, f32x16 (&acc)[4][4],
                                           float (&tot)[4], const float (&ns_a)[4], const float (&ns_b)[4]) {
  constexpr int NB = MODE == kHalfY ? 2 : 4;            // B 32-column blocks of the wave
  constexpr bool kSame = MODE == kFullSumA;             // B fragments = A fragments
  const int64_t N = a.N;
  const int IN = a.IN;
  const int n_steps = (int)((N + kKB - 1) / kKB);
  const uint16_t* Xg = a.X + g * N * IN;
  const uint16_t* Yg = a.Y + g * N * kD;
  const bool b_is_y = tj.b0 == kYTile;

  // ---- copies: wave w issues instructions n = w + 4jj (jj < 8) of each
  // operand; instruction n fills tile rows 2n, 2n+1, lane i row 2n + i/32,
  // slot i % 32, i.e. the piece (i % 32) ^ row_swz(row).  Piece p of an X
  // tile holds features 128 (p < 16 ? g0 : g1) + 8 (p % 16) of its groups;
  // pieces of a missing group, and pieces past 15 of a Y tile, read zeros.
  const int slot_i = lane & 31;
  auto row_of = [&](int jj) __attribute__((always_inline)) { return 2 * (w + 4 * jj) + (lane >> 5); };
  auto x_voff = [&](int jj, int g0, int g1) __attribute__((always_inline)) {
    const int r = row_of(jj), p = slot_i ^ row_swz(r);
    const int gr = p < 16 ? g0 : g1;
    return gr >= 0 ? (uint32_t)r * IN * 2 + 2 * (kGroupW * gr + 8 * (p & 15)) : kSkip;
  };
  auto b_voff = [&](int jj) __attribute__((always_inline)) {
    if (b_is_y) {
      const int r = row_of(jj), p = slot_i ^ row_swz(r);
      return p < kD / 8 ? (uint32_t)r * kD * 2 + 16 * p : kSkip;
    }
    return x_voff(jj, tj.b0, tj.b1);
  };
  // descriptors of step s: the observations from 64 s on (rows past N read zeros)
  auto a_rsrc = [&](int s) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)s * kKB;
    return rsrc_words(Xg + t0 * IN, (uint32_t)((N - t0) * IN * 2));
  };
  auto b_rsrc = [&](int s) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)s * kKB;
    return b_is_y ? rsrc_words(Yg + t0 * kD, (uint32_t)((N - t0) * kD * 2))
                  : rsrc_words(Xg + t0 * IN, (uint32_t)((N - t0) * IN * 2));
  };
  auto copy_one = [&](int p, int q, const u32x4& ra, const u32x4& rb) __attribute__((always_inline)) {
    if (q < kPer)
      dma16(ra, x_voff(q, tj.a0, tj.a1), 0, sm.A[p] + 1024 * (w + 4 * q));
    else
      dma16(rb, b_voff(q - kPer), 0, sm.B[p] + 1024 * (w + 4 * (q - kPer)));
  };

  // ---- fragment reads: lane l (16-lane group gg = l/16: feature half fb =
  // gg%2, k-group kg = gg/2; in the group e = (l%16)/4, q = l%4) names
  // observation row 8kg + e (+ 16ks + 4r) and features 32mb + 16fb + 4q ..
  // +3 of its wave's 128; it receives feature 32mb + 16fb + l%16 (= 32mb +
  // l%32) of 4 rows.  Lanes l and l + 32 hold different observations.
  const int gg = lane >> 4, fb = gg & 1, kg = gg >> 1, e = (lane >> 2) & 3, q4 = lane & 3;
  const int trow = 8 * kg + e;
  const uint32_t row_base = (uint32_t)trow * kRowBytes + 8 * (q4 & 1);
  uint32_t a_off[4], b_off[NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) a_off[mb] = row_base + 16 * ((wj.a_p0 + 4 * mb + 2 * fb + (q4 >> 1)) ^ row_swz(trow));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b_off[nb] = row_base + 16 * ((wj.b_p0 + 4 * nb + 2 * fb + (q4 >> 1)) ^ row_swz(trow));

  // step 0 in flight, then the pipeline: the copies of step s+1 go out
  // between the first half of the products of step s
  {
    const u32x4 ra = a_rsrc(0), rb = b_rsrc(0);
#pragma unroll
    for (int q = 0; q < 2 * kPer; ++q) copy_one(0, q, ra, rb);
  }
  wait_vmcnt<0>();
  lds_barrier();
  constexpr int kStride = NB / 2;   // products per copy in the first half of a step
  // the shift's selectors, held in registers: the compiler would encode
  // (1, 0) as the inline constant 1.0, which the instruction reads as the
  // fp32 bit pattern, i.e. (0, 1)
  uint32_t sel0 = 0x00003f80u, sel1 = 0x3f800000u;
  asm("" : "+v"(sel0), "+v"(sel1));
  const bf16x2 e0 = __builtin_bit_cast(bf16x2, sel0), e1 = __builtin_bit_cast(bf16x2, sel1);
  // one step; MASK: the group's last step, whose observations may end
  // inside it (only shifted fragments need their padding zeroed)
  auto step = [&](int s, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int p = s & 1;
    const bool more = s + 1 < n_steps;
    const int nv = MASK ? (int)(N - (int64_t)s * kKB) : kKB;   // observations of this step
    const u32x4 ra = a_rsrc(more ? s + 1 : s), rb = b_rsrc(more ? s + 1 : s);
    const char* At = sm.A[p];
    const char* Bt = wj.b_in_a ? sm.A[p] : sm.B[p];
    // this step's column sums (added to the totals once per step, so that
    // each total takes N / 64 additions)
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    // fragments of slice ks + 1 are read while the products of slice ks run
    bf16x8 afs[2][4], bfs[2][NB];
    auto read_ks = [&](int ks, bf16x8* af, bf16x8* bfr) __attribute__((always_inline)) {
      if constexpr (MODE != kIdle) {
        const int nvs = MASK ? nv - 16 * ks : 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = read_frag(At, a_off[i], ks);
          if constexpr (SHIFT) af[i] = shift_frag(af[i], ns_a[i], 8 * kg, nvs, e0, e1);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if constexpr (kSame) {
            bfr[i] = af[i];
          } else {
            bfr[i] = read_frag(Bt, b_off[i], ks);
            if constexpr (SHIFT) bfr[i] = shift_frag(bfr[i], ns_b[i], 8 * kg, nvs, e0, e1);
          }
        }
      }
    };
    read_ks(0, afs[0], bfs[0]);
#pragma unroll
    for (int ks = 0; ks < kKB / 16; ++ks) {
      bf16x8* af = afs[ks & 1];
      bf16x8* bfr = bfs[ks & 1];
      if (ks + 1 < kKB / 16) read_ks(ks + 1, afs[(ks + 1) & 1], bfs[(ks + 1) & 1]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if constexpr (MODE != kIdle)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
          if constexpr (MODE == kFullSumA)
            if (nb == 0) part[mb] = frag_sum(af[mb], part[mb]);
          if constexpr (MODE == kFullSumB)
            if (mb == 0) part[nb] = frag_sum(bfr[nb], part[nb]);
          const int m = 4 * NB * ks + NB * mb + nb;   // product index within the step
          if (more && m % kStride == kStride - 1 && m / kStride < 2 * kPer) copy_one(p ^ 1, m / kStride, ra, rb);
        }
    }
    if constexpr (MODE == kFullSumA || MODE == kFullSumB) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] += part[i];
    }
    wait_vmcnt<0>();
    lds_barrier();   // step s+1 landed everywhere; everyone is done with buffer p
  };
  if constexpr (SHIFT) {
    for (int s = 0; s + 1 < n_steps; ++s) step(s, std::false_type());
    step(n_steps - 1, std::true_type());
  } else {
    for (int s = 0; s < n_steps; ++s) step(s, std::false_type());
  }
}

// The per-feature shifts of every group (one thread per X feature or Y
// column): the first observation's value when the first min(N, 64)
// observations share its sign and lie within a factor 1.5 of each other,
// else 0.  Block b covers group b / nb, columns 256 (b % nb) ...
__global__ void __launch_bounds__(kThreads) ridge_shift_kernel(GramArgs a, int32_t nb) {
  const int64_t g = blockIdx.x / nb;
  const int c = (int)(blockIdx.x % nb) * kThreads + threadIdx.x;
  const int IN = a.IN;
  if (c >= IN + kD) return;
  const bool is_x = c < IN;
  const uint16_t* p = is_x ? a.X + g * a.N * IN + c : a.Y + g * a.N * kD + (c - IN);
  const int64_t ld = is_x ? IN : kD;
  const int rows = (int)(a.N < kKB ? a.N : kKB);
  const float first = __uint_as_float((uint32_t)p[0] << 16);
  float lo = first, hi = first;
  for (int r = 1; r < rows; ++r) {
    const float v = __uint_as_float((uint32_t)p[r * ld] << 16);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const bool tight = (lo > 0.f && hi <= 1.5f * lo) || (hi < 0.f && lo >= 1.5f * hi);
  a.shift[g * (IN + kD) + c] = tight ? first : 0.f;
}

__global__ void __launch_bounds__(kThreads, 1) ridge_gram_kernel(GramArgs a) {
  __shared__ GramSmem sm;
  // tile of this workgroup: with groups a multiple of 8, all tiles of group
  // g run on XCD g % 8 (workgroup id mod 8) and share its L2
  const int64_t bid = blockIdx.x;
  int64_t g;
  int t;
  if (a.G % 8 == 0) {
    const int64_t q = bid / 8;
    g = bid % 8 + 8 * (q / a.tiles);
    t = (int)(q % a.tiles);
  } else {
    g = bid / a.tiles;
    t = (int)(bid % a.tiles);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int IN = a.IN;
  TileJob tj;
  WaveJob wj;
  decode_tile(a, t, w, tj, wj);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  float tot[4] = {0.f, 0.f, 0.f, 0.f};
  // minus the shifts of the wave's fragment features: A row 32i + lane%32
  // of its block, B column 32i + lane%32 (a Y column for X^T Y blocks)
  float ns_a[4] = {0.f, 0.f, 0.f, 0.f}, ns_b[4] = {0.f, 0.f, 0.f, 0.f};
  if (wj.mode != kIdle) {
    const float* sh = a.shift + g * (int64_t)(IN + kD);
    const int l32 = lane & 31, nbs = wj.mode == kHalfY ? 2 : 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ns_a[i] = -sh[wj.row0 + 32 * i + l32];
      if (i < nbs) ns_b[i] = -sh[(wj.cross ? IN : 0) + wj.col0 + 32 * i + l32];
    }
  }
  bool nz = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) nz = nz || ns_a[i] != 0.f || ns_b[i] != 0.f;
  const bool shifted = __builtin_amdgcn_ballot_w64(nz) != 0;   // wave-uniform
#define HELM_GRAM(M)                                                                   \
  (shifted ? gram_steps<M, true>(a, sm, g, tj, wj, w, lane, acc, tot, ns_a, ns_b)       \
           : gram_steps<M, false>(a, sm, g, tj, wj, w, lane, acc, tot, ns_a, ns_b))
  switch (wj.mode) {
    case kFull: HELM_GRAM(kFull); break;
    case kFullSumA: HELM_GRAM(kFullSumA); break;
    case kFullSumB: HELM_GRAM(kFullSumB); break;
    case kHalfY: HELM_GRAM(kHalfY); break;
    default: gram_steps<kIdle, false>(a, sm, g, tj, wj, w, lane, acc, tot, ns_a, ns_b); break;
  }
#undef HELM_GRAM

  // ---- epilogue: accumulator register r of a 32 x 32 block holds row
  // 8(r/4) + 4(lane/32) + r%4, column lane%32
  const int col = lane & 31, rgrp = 4 * (lane >> 5);
  if (wj.mode != kIdle) {
    float* out = wj.cross ? a.cross + g * (int64_t)IN * kD : a.gram + g * (int64_t)IN * IN;
    const int64_t ld = wj.cross ? kD : IN;
    const int nbs = wj.mode == kHalfY ? 2 : 4;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        if (nb < nbs) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wj.row0 + 32 * mb + 8 * (r >> 2) + rgrp + (r & 3);
            out[(int64_t)row * ld + wj.col0 + 32 * nb + col] = acc[mb][nb][r];
          }
        }
  }
  if (wj.mode == kFullSumA || wj.mode == kFullSumB) {
    // lanes l and l + 32 summed different observations of column 32i + l%32
    float* sums = a.sums + g * (int64_t)(IN + kD) + wj.sum0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = tot[i] + __shfl_xor(tot[i], 32);
      if (lane < 32) sums[32 * i + lane] = v;
    }
  }
}

// ---------------------------------------------------------------- solve
constexpr int kP = 16;   // panel width of the Cholesky (8 measured slower: twice the passes over M)
constexpr int kRB = 8;   // rows whose memory accesses are issued together

struct SolveArgs {
  const float* gram;     // [G, IN, IN] (upper tiles)
  const float* cross;    // [G, IN, D]
  const float* sums;     // [G, IN + D]
  const float* shift;    // [G, IN + D]
  double* M;             // [G, IN, IN + D] fp64 workspace: upper A | right-hand sides
  float* W;              // [G, IN, D]
  float* b;              // [G, D]
  int64_t N;
  int32_t IN;
  double lambda;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Dynamic LDS of the solve kernel: the panel rows, kP x (IN + D - kP) fp64.
size_t solve_lds_bytes(int32_t IN) { return (size_t)kP * (IN + kD - kP) * sizeof(double); }

// MIN_WAVES: waves per SIMD the register budget must allow.  With IN <= 512
// the kernel's LDS (the panel rows and the diagonal block, unpadded) fits
// twice in a CU, so it is built for two workgroups per CU: two groups'
// memory latency overlap (some registers spill at that budget, and it still
// runs faster).
template <int MIN_WAVES>
__global__ void __launch_bounds__(kThreads, MIN_WAVES) ridge_solve_kernel(SolveArgs a) {
  __shared__ double Dg[kP][kP];
  extern __shared__ double pn_lds[];
  const int64_t g = blockIdx.x;
  const int n = a.IN, ld = n + kD, tid = threadIdx.x;
  const double invN = 1.0 / (double)a.N;
  const float* __restrict__ G = a.gram + g * (int64_t)n * n;
  const float* __restrict__ C = a.cross + g * (int64_t)n * kD;
  const float* __restrict__ sx = a.sums + g * (int64_t)(n + kD);
  const float* __restrict__ sy = sx + n;
  const float* __restrict__ sh = a.shift + g * (int64_t)(n + kD);   // the shifts: mean = shift + sums / N
  double* __restrict__ M = a.M + g * (int64_t)n * ld;
  const int pld = n + kD - kP;   // row length of the panel rows in LDS
  auto Pn = [&](int r, int c) __attribute__((always_inline)) -> double& { return pn_lds[r * pld + c]; };

  // centred normal matrix + lambda I (upper: row j, columns i >= j) and
  // centred right-hand sides X^T Y - sx sy^T / N
  // (rows in batches of kRBs, their loads issued together)
  constexpr int kRBs = 32;
  static_assert(128 % kRBs == 0, "input widths are multiples of 128");
  for (int j0 = 0; j0 < n; j0 += kRBs) {
    for (int i = j0 + tid; i < ld; i += kThreads) {
      const bool a_part = i < n;
      const double si = a_part ? (double)sx[i] : (double)sy[i - n];
      float raw[kRBs];
#pragma unroll
      for (int u = 0; u < kRBs; ++u)
        raw[u] = a_part ? (i >= j0 + u ? G[(int64_t)(j0 + u) * n + i] : 0.0f) : C[(int64_t)(j0 + u) * kD + (i - n)];
#pragma unroll
      for (int u = 0; u < kRBs; ++u) {
        const int j = j0 + u;
        if (!a_part || i >= j)
          M[(int64_t)j * ld + i] = (double)raw[u] - (double)sx[j] * si * invN + (i == j ? a.lambda : 0.0);
      }
    }
  }
  __syncthreads();

  // ---- A = U^T U, forward substitution U^T Z = B folded in: panel k0
  for (int k0 = 0; k0 < n; k0 += kP) {
    // diagonal block, factored in LDS
    for (int e = tid; e < kP * kP; e += kThreads) {
      const int r = e / kP, c = e % kP;
      if (c >= r) Dg[r][c] = M[(int64_t)(k0 + r) * ld + k0 + c];
    }
    __syncthreads();
    // (by wave 0 alone: one wave's LDS accesses take effect in issue order,
    // so a compiler barrier orders its lanes' steps)
    if (tid < 64) {
      for (int r = 0; r < kP; ++r) {
        const double piv = sqrt(Dg[r][r]);   // a non-positive pivot gives NaN
        wave_sync();
        if (tid == r)
          Dg[r][r] = piv;
        else if (tid > r && tid < kP)
          Dg[r][tid] /= piv;
        wave_sync();
        for (int e = tid; e < kP * kP; e += 64) {
          const int s = e / kP, c = e % kP;
          if (s > r && c >= s) Dg[s][c] -= Dg[r][s] * Dg[r][c];
        }
        wave_sync();
      }
    }
    __syncthreads();
    for (int e = tid; e < kP * kP; e += kThreads) {
      const int r = e / kP, c = e % kP;
      if (c >= r) M[(int64_t)(k0 + r) * ld + k0 + c] = Dg[r][c];
    }
    // panel rows k0 .. k0+15, columns past the block (the rest of U's rows
    // and the right-hand sides): solve U_kk^T X = panel, one column a thread
    const int m0 = k0 + kP, width = ld - m0;
    for (int c = tid; c < width; c += kThreads) {
      // the diagonal block is read anew for each column (an opaque offset):
      // hoisted out of the loop, its 136 values would hold registers
      int dz = 0;
      asm volatile("" : "+v"(dz));
      const double* dg = &Dg[0][0] + dz;
      double x[kP];
#pragma unroll
      for (int r = 0; r < kP; ++r) {
        double v = M[(int64_t)(k0 + r) * ld + m0 + c];
#pragma unroll
        for (int p = 0; p < r; ++p) v -= dg[p * kP + r] * x[p];
        x[r] = v / dg[r * kP + r];
      }
#pragma unroll
      for (int r = 0; r < kP; ++r) {
        Pn(r, c) = x[r];
        M[(int64_t)(k0 + r) * ld + m0 + c] = x[r];
      }
    }
    __syncthreads();
    // trailing update: row s >= m0, column j >= s (A part) or any column of
    // the right-hand sides: M[s][j] -= sum_r Pn[r][s - m0] Pn[r][j - m0]
    // (rows in batches of kRB, their loads issued together)
    for (int c = tid; c < width; c += kThreads) {
      const int j = m0 + c;
      double col[kP];
#pragma unroll
      for (int r = 0; r < kP; ++r) col[r] = Pn(r, c);
      const int s_stop = (j < n ? j : n - 1) + 1;
      int s = m0;
      for (; s + kRB <= s_stop; s += kRB) {
        double mv[kRB];
#pragma unroll
        for (int u = 0; u < kRB; ++u) mv[u] = M[(int64_t)(s + u) * ld + j];
#pragma unroll
        for (int u = 0; u < kRB; ++u) {
          double v = 0.0;
#pragma unroll
          for (int r = 0; r < kP; ++r) v += Pn(r, s + u - m0) * col[r];
          M[(int64_t)(s + u) * ld + j] = mv[u] - v;
        }
      }
      for (; s < s_stop; ++s) {
        double v = 0.0;
#pragma unroll
        for (int r = 0; r < kP; ++r) v += Pn(r, s - m0) * col[r];
        M[(int64_t)s * ld + j] -= v;
      }
    }
    __syncthreads();
  }

  // ---- back substitution U W = Z, panels from the last: W_K from the
  // diagonal block, then Z rows above it lose U[j][K] W_K.  The panel's
  // column block of U above the diagonal (rows j < k0) is staged in the
  // panel rows' LDS as Pn(r, kD + j) = U[j][k0 + r], read back by every
  // lane of a wave at once.
  for (int k0 = ((n - 1) / kP) * kP; k0 >= 0; k0 -= kP) {
    for (int e = tid; e < kP * kP; e += kThreads) {
      const int r = e / kP, c = e % kP;
      if (c >= r) Dg[r][c] = M[(int64_t)(k0 + r) * ld + k0 + c];
    }
    for (int e0 = tid; e0 < k0 * kP; e0 += kRB * kThreads) {
      double t[kRB];
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const int e = e0 + u * kThreads;
        t[u] = e < k0 * kP ? M[(int64_t)(e / kP) * ld + k0 + e % kP] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const int e = e0 + u * kThreads;
        if (e < k0 * kP) Pn(e % kP, kD + e / kP) = t[u];
      }
    }
    __syncthreads();
    if (tid < kD) {
      double wv[kP];
#pragma unroll
      for (int r = kP - 1; r >= 0; --r) {
        double v = M[(int64_t)(k0 + r) * ld + n + tid];
#pragma unroll
        for (int p = r + 1; p < kP; ++p) v -= Dg[r][p] * wv[p];
        wv[r] = v / Dg[r][r];
      }
#pragma unroll
      for (int r = 0; r < kP; ++r) {
        M[(int64_t)(k0 + r) * ld + n + tid] = wv[r];
        Pn(r, tid) = wv[r];
      }
    }
    __syncthreads();
    // rows j < k0: two threads per right-hand column, rows split in halves
    {
      const int d = tid % kD, half = tid / kD;
      double wv[kP];
#pragma unroll
      for (int r = 0; r < kP; ++r) wv[r] = Pn(r, d);
      // (rows in batches of kRB, their loads issued together; k0 is a
      // multiple of kRB, the two halves take alternate batches)
      for (int j0 = half * kRB; j0 < k0; j0 += 2 * kRB) {
        double mv[kRB], v[kRB];
#pragma unroll
        for (int u = 0; u < kRB; ++u) {
          mv[u] = M[(int64_t)(j0 + u) * ld + n + d];
          v[u] = 0.0;
        }
#pragma unroll
        for (int r = 0; r < kP; ++r)
#pragma unroll
          for (int u = 0; u < kRB; ++u) v[u] += Pn(r, kD + j0 + u) * wv[r];
#pragma unroll
        for (int u = 0; u < kRB; ++u) M[(int64_t)(j0 + u) * ld + n + d] = mv[u] - v[u];
      }
    }
    __syncthreads();
  }

  // ---- outputs: W in fp32; b = mean(Y) - mean(X) W in fp64, the means
  // being the shifts plus the shifted data's sums / N
  float* Wg = a.W + g * (int64_t)n * kD;
  for (int e = tid; e < n * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    Wg[e] = (float)M[(int64_t)i * ld + n + d];
  }
  if (tid < kD) {
    double v = (double)sh[n + tid] + (double)sy[tid] * invN;
    for (int i0 = 0; i0 < n; i0 += kRB) {   // (n is a multiple of kRB)
      double mv[kRB];
#pragma unroll
      for (int u = 0; u < kRB; ++u) mv[u] = M[(int64_t)(i0 + u) * ld + n + tid];
#pragma unroll
      for (int u = 0; u < kRB; ++u) v -= ((double)sh[i0 + u] + (double)sx[i0 + u] * invN) * mv[u];
    }
    a.b[g * kD + tid] = (float)v;
  }
}

}  // namespace

int64_t ridge_tiles_per_group(int32_t IN) {
  const int64_t nF = IN / kGroupW, nD = (nF + 1) / 2;
  return nD + nD * (nD - 1) / 2 + (nF / 2 + 1) / 2;
}

bool ridge_supports(const RidgeFit& f) {
  auto al = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
  return f.D == kD && f.IN >= 128 && f.IN <= kMaxIn && f.IN % 128 == 0 && f.N >= 1 &&
         f.N * f.IN * 2 <= (int64_t)kSkip && f.G >= 1 && f.G <= 0x7fffffffLL / ridge_tiles_per_group(f.IN) &&
         al(f.X) && al(f.Y);
}

hipError_t launch_ridge(const RidgeFit& f, bool gram, bool solve, hipStream_t stream) {
  if (!ridge_supports(f)) return hipErrorNotSupported;
  if (gram) {
    GramArgs a{};
    a.X = (const uint16_t*)f.X;
    a.Y = (const uint16_t*)f.Y;
    a.shift = f.shift;
    a.gram = f.gram;
    a.cross = f.cross;
    a.sums = f.sums;
    a.N = f.N;
    a.G = (int32_t)f.G;
    a.IN = f.IN;
    a.nF = f.IN / kGroupW;
    a.tiles = (int32_t)ridge_tiles_per_group(f.IN);
    const int32_t nb = (f.IN + kD + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(ridge_shift_kernel, dim3((unsigned)(f.G * nb)), dim3(kThreads), 0, stream, a, nb);
    hipLaunchKernelGGL(ridge_gram_kernel, dim3((unsigned)(f.G * a.tiles)), dim3(kThreads), 0, stream, a);
  }
  if (solve) {
    SolveArgs s{};
    s.gram = f.gram;
    s.cross = f.cross;
    s.sums = f.sums;
    s.shift = f.shift;
    s.M = f.M;
    s.W = f.W;
    s.b = f.b;
    s.N = f.N;
    s.IN = f.IN;
    s.lambda = f.lambda;
    const size_t lds = solve_lds_bytes(f.IN);
    const bool two = lds + sizeof(double) * kP * kP <= 80 * 1024;   // two workgroups' LDS in one CU
    const void* fn = two ? (const void*)ridge_solve_kernel<2> : (const void*)ridge_solve_kernel<1>;
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    if (two)
      hipLaunchKernelGGL(ridge_solve_kernel<2>, dim3((unsigned)f.G), dim3(kThreads), lds, stream, s);
    else
      hipLaunchKernelGGL(ridge_solve_kernel<1>, dim3((unsigned)f.G), dim3(kThreads), lds, stream, s);
  }
  return hipGetLastError();
}

}  // namespace helm
