// stream_big.hip -- matrix products of the streamed path for large slices in
// bf16 mode (m >= 129, dimensions padded to multiples of 256).
//
// Per Newton-Schulz round ("关于分布式Muon的想法整合及讨论" §2 and §6: the Gram
// matrix is recomputed each round; "MindSpore HyperParallel X 盘古,Muon优化器实现
// 6倍性能跃升", 三大性能挑战: the round is matrix products and additions):
//
//   gram   A = s2 X X^T, stored three ways: float32 A (tiles on and above
//          the diagonal), the diagonal d = diag(A) in float32, and
//          E = A - diag(d) rounded to bf16 (the operand of the next product);
//   poly   R = (a - 1) I + b A + c A^2 with
//            A^2 = E E + diag(d) A + A diag(d) - diag(d)^2,
//          where only E E runs on the matrix cores; R is rounded to bf16;
//   apply  X' = s (X + R X) = s (a X + (b A + c A^2) X); the X term is added
//          to the float32 accumulators from the X^T operand slices already
//          in LDS (bf16 X is exact in float32), so the epilogue reads no X.
//
// Keeping the diagonal out of the bf16 operands and shifting the polynomial by
// the identity leaves bf16 rounding only on the small off-diagonal part of A
// and on R, whose spectrum is near zero once the iteration has converged.
// This is an arithmetic arrangement of the same iteration, not a different
// method.
//
// The kernel: 256 x 256 output tile per 512-thread workgroup, eight waves
// in a 2 x 4 grid each owning 128 x 64 (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16).  Two waves share each SIMD, so one wave's
// matrix-core products run while the other waits on LDS or the barrier;
// with one wave per SIMD (four waves of 128 x 128) the products ran about
// 12% slower.
// Operand k-slices of kBK elements go from HBM straight into LDS with
// gfx950's global_load_lds_dwordx4, kNS stages deep with one barrier per
// slice; lane l of a load lands at byte 16 l of its 1 KB destination, and
// each lane fetches the 16-byte chunk of its row that belongs in its slot
// under the XOR swizzle below, so the 16-byte fragment reads of 16
// consecutive rows hit distinct bank groups.  (Measured on the large
// workloads: 64-element slices in 2 stages, 32 in 3 and 32 in 4 are within
// 2% of each other; the matrix cores, not load latency, set the pace.)
// One launch per phase covers every large bucket.  Output tiles come from a
// table that the planner builds: workgroups are dealt to the 8 XCDs round
// robin, so workgroup b takes entry (b mod 8) * T/8 + b/8 and XCD x walks the
// x-th stretch of the table.  Each stretch holds whole blocks of 4 x 8 tiles
// (the 32 workgroups an XCD runs at once share 4 row and 8 column panels in
// its L2), longest contraction first, with the work balanced over the XCDs.
// Symmetric products (X X^T, E E) list only tiles on or above the diagonal
// (on slices with a padded last tile row they compute the mirrors below it);
// the bf16 result of an off-diagonal tile is also written to its mirror
// position.  A tile of a last tile row with at most 128 rows inside m is a
// half tile: it computes those 128 rows only, the eight waves taking 64 x 64
// each.  The
// epilogue turns the accumulators around in LDS and writes
// whole rows of 16-byte pieces.  Where a transposed copy holds the same values
// (the mirror tiles, and X'^T next to X'), it is read out of LDS after the
// row-view results, so the side inputs of the epilogue are read only once.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

constexpr int kBK = kBigKStep;               // bf16 elements of k per slice
constexpr int kNS = 2;                       // LDS stages (slices in flight: kNS - 1)
constexpr int kRB = 2 * kBK;                 // bytes of one tile row per slice
constexpr int kCPR = kRB / 16;               // 16-byte chunks per row
constexpr int kRPI = 1024 / kRB;             // rows filled by one 1 KB load instruction
constexpr int kRW = 256 / kRB;               // rows per 256-byte span of the LDS banks
constexpr int kWavesBig = 8;                 // waves per workgroup: 2 along i, 4 along j
constexpr int kThreadsBig = 64 * kWavesBig;
constexpr int kLI = kBigTile / kRPI / kWavesBig;  // load instructions per wave, operand and slice
constexpr int kStage = 2 * kBigTile * kRB;   // bytes per stage (A and B tiles)
constexpr int kNSHalf = 3;                   // LDS stages of a half tile's loop
constexpr int kStageHalf = (128 + kBigTile) * kRB;  // its stage: 128 rows of A, 256 of B
constexpr int kStageBytes = 128 * 256 * 4;   // epilogue staging: 128 rows of 256 floats
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kLds = cmax(cmax(kNS * kStage, kNSHalf * kStageHalf), kStageBytes);
constexpr int kViewRow = 1, kViewCol = 2;
static_assert(kBK % 16 == 0 && kCPR <= 8 && kNS >= 2 && kNSHalf >= 2 && kLds <= 160 * 1024 && kLI % 2 == 0,
              "tile geometry");

#define LDS_PTR __attribute__((address_space(3)))

// Chunk c of tile row r sits in LDS slot c ^ swz(r): the 16 rows that one
// 16-lane group of a fragment read touches then cover 16 distinct 16-byte
// bank groups.
__device__ __forceinline__ int swz(int r) { return (r / kRW) & (kCPR - 1); }

// Epilogue staging of the row view (128 rows of 256 float32): the 16-byte
// slot s of row r sits at s ^ stage_swz(r).  Bit 3 follows r / 4, so the
// two half-waves of an accumulator write (rows r and r + 4) fill disjoint
// halves of the banks; the low bits follow r / 8, so the rows 8 k + u that
// the transposed readout gathers at once sit in distinct slots.
__device__ __forceinline__ int stage_swz(int r) { return ((r >> 3) & 15) ^ (((r >> 2) & 1) << 3); }

// Wait until at most `slices` k-slices of this wave's operand loads (L load
// instructions per slice) are in flight.
template <int L>
__device__ __forceinline__ void wait_loads(int slices) {
  static_assert(kNS - 2 <= 3 && kNSHalf - 2 <= 3 && 3 * L < 64, "extend the cases");
  switch (slices) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * L) : "memory"); break;
  }
}

__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Operands of one tile's product: rows of A and of B are contiguous along k.
struct Operands {
  const char* a;
  const char* b;
  int64_t lda, ldb, K;
};

__device__ __forceinline__ void st_bf16x4(uint16_t* p, f32x4_t v) {
  *reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(p)) =
      u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
__device__ __forceinline__ f32x4_t ld_f32x4(const float* p) {
  return *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(p));
}
__device__ __forceinline__ void st_f32x4(float* p, f32x4_t v) {
  *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(p)) = v;
}

template <class Epi>
__global__ __launch_bounds__(kThreadsBig) void k_gemm_big(BigArgs g) {
  constexpr int FM = 4, FN = 2;    // 32x32 blocks per wave along i and j
  __shared__ __attribute__((aligned(1024))) char lds[kLds];

  int b = blockIdx.x;
  b = (b & 7) * (g.t8 >> 3) + (b >> 3);
  const BigTile t = g.tiles[b];
  if (t.bz == kNoTile) return;  // uniform over the workgroup, before any barrier
  const BigBucket& bb = g.buckets[t.bz >> 24];  // read in place: fields are indexed by round parity
  const int z = (int)(t.bz & 0xFFFFFFu);
  // The table lists a symmetric product's tiles on and above the diagonal.
  // On a slice whose m is not a multiple of the tile, Epi::kLower phases
  // compute the mirror tile below it instead (the transposed copy goes out
  // through the mirror writes), so that the padded last tile row, not
  // column, holds the rows past m.
  const int t_i = (int)(t.mn & 0xFFFFu), t_j = (int)(t.mn >> 16);
  const bool lower = Epi::kLower && bb.m % kBigTile != 0;
  const int tm = lower ? t_j : t_i, tn = lower ? t_i : t_j;
  const Operands op = Epi::operands(g, bb, z);
  // The epilogue's context (table reads for the final phase) is fetched
  // here, so its loads complete during the products.
  const auto cx = Epi::context(g, bb, z);

  const int tid = threadIdx.x, lane = tid & 63;
  // The wave index is uniform over the wave; saying so keeps branches on it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // Half tiles (the symmetric products).  X and E are zero in their rows
  // past m, and so are X X^T and E E.  In the last tile row of a slice with
  // at most 128 real rows there (the phases' padded row, Epi::kLower), the
  // tile's rows 128..255 are therefore zero, which the workspace already
  // holds (it is cleared once, and nothing writes anything else there).
  // Such a tile computes its first 128 rows only: the eight waves take
  // 64 x 64 each (2 x 2 blocks) instead of 128 x 64 (4 x 2), only those 128
  // rows of the first operand are loaded, and the epilogue writes one half.
  // It takes about 60% of a full tile's time (fewer products per k-slice
  // hide less of each slice's fixed cost), in the same launch as the full
  // tiles, which fills the last wave of tiles better.  (The apply and final
  // phases have none: on launches that fill the chip their half tiles were
  // no faster, and with them in the kernel the compiler's code for the full
  // tiles' X term, further down, ran up to 1% slower.)
  const bool half = Epi::kLower && bb.m - (int64_t)tm * kBigTile <= 128;
  // The symmetric products are zero in their columns past m as well: on a
  // half tile on the diagonal, a wave whose 64 columns all lie past m skips
  // its products, and its accumulators keep the zero they would give.
  const bool idle = Epi::kLower && half && (int64_t)tn * kBigTile + wn * 64 >= bb.m;
  const char* A = op.a + (int64_t)tm * kBigTile * op.lda * 2;
  const char* B = op.b + (int64_t)tn * kBigTile * op.ldb * 2;
  const int nk = (int)(op.K / kBK);

  // Load instruction u of wave w fills rows kRPI (w + 8 u) .. + kRPI - 1 of an
  // operand tile; lane l lands in slot l mod kCPR of row l / kCPR and fetches
  // the chunk that belongs there.
  uint32_t oa[kLI], ob[kLI];
#pragma unroll
  for (int u = 0; u < kLI; ++u) {
    const int row = kRPI * (wave + kWavesBig * u) + lane / kCPR;
    const int chunk = (lane % kCPR) ^ swz(row);
    oa[u] = (uint32_t)(row * op.lda * 2 + chunk * 16);
    ob[u] = (uint32_t)(row * op.ldb * 2 + chunk * 16);
  }
  // A half tile loads rows 0..127 of the first operand only (u < kLI / 2),
  // into stages of its own size (B at stage row 128), kNSHalf deep: with
  // half the products per slice, one slice in flight left its loop waiting
  // on the loads.  The swizzle of B-stage row 128 + r (or 256 + r) equals
  // that of operand row r.
  auto issue = [&](int kt, int stage, auto half_tag) {
    constexpr bool H = decltype(half_tag)::value;
    constexpr int kLA = H ? kLI / 2 : kLI;
    constexpr int kStg = H ? kStageHalf : kStage;
    constexpr int kOffB = (H ? 128 : kBigTile) * kRB;
    char LDS_PTR* base = (char LDS_PTR*)(lds + stage * kStg);
#pragma unroll
    for (int u = 0; u < kLA; ++u)
      __builtin_amdgcn_global_load_lds((const MUON_GLOBAL void*)(A + (int64_t)kt * kRB + oa[u]),
                                       (void LDS_PTR*)(base + (wave + kWavesBig * u) * 1024), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < kLI; ++u)
      __builtin_amdgcn_global_load_lds((const MUON_GLOBAL void*)(B + (int64_t)kt * kRB + ob[u]),
                                       (void LDS_PTR*)(base + kOffB + (wave + kWavesBig * u) * 1024), 16, 0, 0);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  // Multiply one resident slice.  The fragments of k-substep s + 1 are read
  // from LDS while the products of substep s run (two fragment sets), and
  // the scheduling hints interleave one fragment read with every product
  // or two, so the matrix cores are not left waiting on LDS.  A half tile's
  // wave takes the first FM / 2 blocks of its accumulators, rows 64 wm ..
  // + 63 of the tile.
  constexpr int kSub = kBK / 16;
  auto multiply = [&](const char* st, auto half_tag) {
    constexpr bool H = decltype(half_tag)::value;
    constexpr int F = H ? FM / 2 : FM;
    const int ra = (H ? wm * 64 : wm * 128) + (lane & 31);
    const int rb = (H ? 128 : kBigTile) + wn * 64 + (lane & 31);
    bf16x8_t af[2][F], bfr[2][FN];
    auto fragments = [&](int s, int buf) {
      const int ck = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int r = ra + 32 * i;
        af[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + r * kRB + ((ck ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = rb + 32 * j;
        bfr[buf][j] = *reinterpret_cast<const bf16x8_t*>(st + r * kRB + ((ck ^ swz(r)) << 4));
      }
    };
    fragments(0, 0);
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      if (s + 1 < kSub) fragments(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(af[s & 1][i], bfr[s & 1][j], acc[i][j]);
    }
    // Order: the first substep's F + FN reads, then (1 product, 1 read)
    // F + FN times and the remaining products per following substep, then
    // the last substep's F FN products.
    __builtin_amdgcn_sched_group_barrier(0x100, F + FN, 0);
#pragma unroll
    for (int s = 0; s + 1 < kSub; ++s) {
#pragma unroll
      for (int q = 0; q < F + FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (F * FN > F + FN) __builtin_amdgcn_sched_group_barrier(0x008, F * FN - (F + FN), 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, F * FN, 0);
  };

  // Epi::kAddX (X + R X, second operand X^T): the k-slices whose k range is
  // this tile's own row range hold X at exactly the entries of the output
  // tile (B-stage row j, k = i holds X[i][j]), so the waves whose rows they
  // are add them to their accumulators and the epilogue reads no X.  Slice
  // kt covers tile rows 64 (kt mod 4) .. + 63, rows 64 (kt mod 2) .. + 63 of
  // the waves with wm = (kt mod 4) / 2: their 32-row blocks I0 = 2 (kt mod 2)
  // and I0 + 1.  Register 4 q + e of block I0 + ii is row
  // 32 ii + 8 q + 4 (l / 32) + e of the slice, column l mod 32: four
  // consecutive k of B-stage row rb + 32 j, one 8-byte read.  (I0 is a
  // constant, so the accumulators stay in registers.)
  auto add_x = [&](const char* st, int rb, auto i0_tag) {
    constexpr int I0 = decltype(i0_tag)::value;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rb + 32 * j, ck = 4 * ii + q;
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(st + r * kRB + ((ck ^ swz(r)) << 4) + 8 * (lane >> 5));
          acc[I0 + ii][j][4 * q + 0] += bf16_lo(v.x);
          acc[I0 + ii][j][4 * q + 1] += bf16_hi(v.x);
          acc[I0 + ii][j][4 * q + 2] += bf16_lo(v.y);
          acc[I0 + ii][j][4 * q + 3] += bf16_hi(v.y);
        }
  };

  // NS - 1 slices in flight (NS = kNS, or kNSHalf on a half tile).
  // Iteration kt: wait for this wave's loads of slice kt; one barrier then
  // says that every wave's part of slice kt is in LDS and that every wave
  // has finished reading slice kt - 1, whose stage is refilled with slice
  // kt + NS - 1 before slice kt is multiplied.  (One loop: peeling the last
  // slices off made the compiler spill the accumulators around the
  // epilogue.)  The symmetric products run this loop, one copy for full and
  // one for half tiles, chosen once per workgroup.  The apply phases run the
  // same loop with the X term, written out in the kernel body below: inside
  // a lambda, which is optimized before it is inlined, the X term's two
  // calls were merged into one through a pointer, and the accumulators
  // stayed on the stack.
  auto main_loop = [&](auto half_tag) {
    constexpr bool H = decltype(half_tag)::value;
    constexpr int NS = H ? kNSHalf : kNS;
    constexpr int kStg = H ? kStageHalf : kStage;
    constexpr int L = (H ? kLI / 2 : kLI) + kLI;  // load instructions per slice and wave
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < nk) issue(p, p, half_tag);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_loads<L>(min(NS - 2, nk - 1 - kt));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");  // no LDS access moves across the barrier
      if (kt + NS - 1 < nk) issue(kt + NS - 1, stage == 0 ? NS - 1 : stage - 1, half_tag);
      if constexpr (H) {
        if (!idle) multiply(lds + stage * kStg, half_tag);
      } else {
        multiply(lds + stage * kStg, half_tag);
      }
      stage = stage == NS - 1 ? 0 : stage + 1;
    }
  };

  // ---- epilogue.  Accumulator layout of a 32x32 block: lane l, register r ->
  // row 8 (r / 4) + 4 (l / 32) + r mod 4, column l mod 32.  One pass stages
  // 128 rows of the tile (128 x 256 float32 = 128 KB) and writes them as
  // whole rows of 16-byte pieces: two passes for a full tile, one for a half
  // tile.  What an epilogue reads besides the product (W, A, the diagonal)
  // is loaded kBatch pieces at a time, the first batch before the staging
  // so its latency is hidden.
  // A phase whose transposed output holds the same values as its own
  // (Epi::kMirror: the symmetric products, and X' next to X'^T) computes
  // them once, in the row view: each thread puts its results back into the
  // staging slots it read them from, and the transposed rows are then read
  // out of LDS down the columns, 8 values (16 bytes of bf16) per thread.
  // Such a phase reads its side inputs in one layout only.
  const int views = Epi::views(cx, tm == tn);
  const bool mirror = Epi::kMirror && (views & kViewCol);
  const float pre = Epi::prescale(cx);
  float* stg = reinterpret_cast<float*>(lds);
  auto pass = [&](auto view_tag, auto half_tag, auto ht_tag) {
    constexpr bool HT = decltype(ht_tag)::value;  // a half tile
    constexpr int V = decltype(view_tag)::value;
    constexpr int h = decltype(half_tag)::value;
    constexpr int kPieces = 128 * 64 / kThreadsBig;  // 16-byte pieces of one pass (128 rows) per thread
    // In the second half every wave has staged its accumulators before the
    // side inputs are loaded, so their registers can hold a larger batch
    // (Epi::kBatchLast) of those loads; the first half loads its first batch
    // ahead of the staging, to hide its latency.
    constexpr bool late = h == 1 && Epi::kBatchLast > Epi::kBatch;
    constexpr int kB = late ? Epi::kBatchLast : Epi::kBatch;
    constexpr int NB = kB < kPieces ? kB : kPieces;
    const int row0 = (V == kViewRow ? tm : tn) * kBigTile + h * 128;
    const int col0 = (V == kViewRow ? tn : tm) * kBigTile;
    // Epi::kFastPath: where this pass's 128 rows lie wholly inside the side
    // input's storage (uniform over the workgroup), the loads and stores run
    // in a copy of the loop without per-lane guards, chosen once per pass:
    // guards around each load make the compiler wait for it at once, so a
    // batch's loads would not be in flight together.
    using Guarded = std::false_type;
    using Unguarded = std::true_type;
    bool fast = false;
    if constexpr (Epi::kFastPath) fast = Epi::fast(cx, V, row0, col0);
    typename Epi::Aux aux[NB];
    auto load_batch = [&](int b0, auto fast_tag) {
      constexpr bool kF = decltype(fast_tag)::value;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int idx = (b0 + u) * kThreadsBig + tid;
        aux[u] = Epi::template load<kF>(cx, V, row0 + (idx >> 6), col0 + 4 * (idx & 63));
      }
    };
    auto first_batch = [&] {
      if constexpr (Epi::kFastPath) {
        if (fast) load_batch(0, Unguarded{});
        else load_batch(0, Guarded{});
      } else {
        load_batch(0, Guarded{});
      }
    };
    if constexpr (!late) first_batch();
    if constexpr (V == kViewRow) {
      // Staged [i][j]; 16-byte slot s of row r sits at s ^ stage_swz(r).
      // A full tile's half h is the rows of the waves with wm = h; a half
      // tile (h = 0 only) has rows 64 wm + 32 i + .., i < FM / 2, in every wave.
      if (HT || wm == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (HT && i >= FM / 2) continue;
                const int r = (HT ? wm * 64 : 0) + i * 32 + 8 * q + 4 * (lane >> 5) + u;
                const int col = wn * 64 + j * 32 + (lane & 31);
                const int ps = (col >> 2) ^ stage_swz(r);
                stg[r * 256 + ps * 4 + (col & 3)] = pre * acc[i][j][4 * q + u];
              }
      }
    } else {
      // Staged [j][i] (four consecutive i per lane are one 16-byte slot);
      // slot s of row r sits at s ^ (r mod 16).  On a half tile only
      // i < 128 is staged; the rest of each row is past m, where the
      // epilogue's guards store nothing (the tile is never on its fast path).
      if ((wn >> 1) == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (HT && i >= FM / 2) continue;
              const int rc = (wn & 1) * 64 + j * 32 + (lane & 31);
              const int ci = (HT ? wm * 64 : wm * 128) + i * 32 + 8 * q + 4 * (lane >> 5);
              const int ps = (ci >> 2) ^ (rc & 15);
              f32x4_t v;
              v.x = pre * acc[i][j][4 * q + 0];
              v.y = pre * acc[i][j][4 * q + 1];
              v.z = pre * acc[i][j][4 * q + 2];
              v.w = pre * acc[i][j][4 * q + 3];
              *reinterpret_cast<f32x4_t*>(stg + rc * 256 + ps * 4) = v;
            }
      }
    }
    __syncthreads();
    if constexpr (late) first_batch();
    auto batches = [&](auto fast_tag) {
      constexpr bool kF = decltype(fast_tag)::value;
#pragma unroll
      for (int b0 = 0; b0 < kPieces; b0 += NB) {
        if (b0 > 0) load_batch(b0, fast_tag);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int idx = (b0 + u) * kThreadsBig + tid;
          const int r = idx >> 6, sl = idx & 63;
          const int ps = V == kViewRow ? sl ^ stage_swz(r) : sl ^ (r & 15);
          f32x4_t* slot = reinterpret_cast<f32x4_t*>(stg + r * 256 + ps * 4);
          const f32x4_t res = Epi::template store<kF>(cx, V, row0 + r, col0 + 4 * sl, *slot, aux[u]);
          if constexpr (V == kViewRow && Epi::kMirror) {
            if (mirror) *slot = res;
          }
        }
      }
    };
    if constexpr (Epi::kFastPath) {
      if (fast) batches(Unguarded{});
      else batches(Guarded{});
    } else {
      batches(Guarded{});
    }
    __syncthreads();
    if constexpr (V == kViewRow && Epi::kMirror) {
      if (!mirror) return;
      // Transposed rows: in step t wave w takes tile columns 32 w + 4 t ..
      // + 3; lane l takes column j = (l / 8) mod 4 of them and reads rows
      // 8 k .. + 7 of this half down it, k = l mod 8 + 8 (l / 32), writing
      // them as one 16-byte piece of row (column) c.  Each half-wave then
      // gathers 8 row groups x 4 columns, whole 16-byte slots in 8 (16 for
      // the wave) distinct positions, and each column's 16 lanes write 256
      // contiguous bytes.
      const int r0 = 8 * ((lane & 7) + 8 * (lane >> 5));
#pragma unroll 2
      for (int t = 0; t < 8; ++t) {
        const int c = 32 * wave + 4 * t + ((lane >> 3) & 3);
        float e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = r0 + u;
          e[u] = stg[r * 256 + 4 * ((c >> 2) ^ stage_swz(r)) + (c & 3)];
        }
        Epi::store_t(cx, tn * kBigTile + c, tm * kBigTile + h * 128 + r0,
                     u32x4_t{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                             pack_bf16x2(e[6], e[7])});
      }
      __syncthreads();
    }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  using Row = std::integral_constant<int, kViewRow>;
  using Col = std::integral_constant<int, kViewCol>;
  auto epilogue = [&](auto ht) {
    if (views & kViewRow) {
      pass(Row{}, H0{}, ht);
      if constexpr (!decltype(ht)::value) pass(Row{}, H1{}, ht);
    }
    if ((views & kViewCol) && !mirror) {
      pass(Col{}, H0{}, ht);
      pass(Col{}, H1{}, ht);
    }
  };
  using Full = std::false_type;
  using Half = std::true_type;
  if constexpr (Epi::kAddX) {
    const int rb = kBigTile + wn * 64 + (lane & 31);
#pragma unroll
    for (int p = 0; p < kNS - 1; ++p)
      if (p < nk) issue(p, p, Full{});
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_loads<2 * kLI>(min(kNS - 2, nk - 1 - kt));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");  // no LDS access moves across the barrier
      if (kt + kNS - 1 < nk) issue(kt + kNS - 1, stage == 0 ? kNS - 1 : stage - 1, Full{});
      if ((kt >> 2) == tm && wm == ((kt & 3) >> 1)) {
        if (kt & 1) add_x(lds + stage * kStage, rb, std::integral_constant<int, 2>{});
        else add_x(lds + stage * kStage, rb, std::integral_constant<int, 0>{});
      }
      multiply(lds + stage * kStage, Full{});
      stage = stage == kNS - 1 ? 0 : stage + 1;
    }
    __syncthreads();  // every wave is done with the stages before they hold the epilogue
    epilogue(Full{});
  } else if (half) {
    main_loop(Half{});
    __syncthreads();
    epilogue(Half{});
  } else {
    main_loop(Full{});
    __syncthreads();
    epilogue(Full{});
  }
}

// ------------------------------------------------------------------ epilogues
// Each phase supplies its operands and an epilogue.  load(cx, view, r, c)
// fetches what the epilogue needs besides the product for entries
// (r, c .. c+3) of the output in the given view (kViewCol: of the transposed
// output), c a multiple of 4; store(cx, view, r, c, v, aux) writes them.

__device__ __forceinline__ f32x4_t ld_bf16x4(const uint16_t* p) {
  const u32x2_t w = *reinterpret_cast<const MUON_GLOBAL u32x2_t*>(as_global(p));
  return f32x4_t{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
}

// A = s2 X X^T: float32 A, float32 diagonal, bf16 A with a zero diagonal.
struct GramPhase {
  static __device__ Operands operands(const BigArgs& g, const BigBucket& bb, int z) {
    const char* x = bb.x[g.src] + (int64_t)z * bb.mp * bb.np * 2;
    return Operands{x, x, bb.np, bb.np, big_k_over_m(bb.n)};
  }
  struct Ctx {
    float* a32;
    uint16_t* e16;
    float* dg;
    int64_t mp;
    float pre;
  };
  static __device__ Ctx context(const BigArgs& g, const BigBucket& bb, int z) {
    const int64_t o = (int64_t)z * bb.mp * bb.mp;
    return Ctx{bb.a32 + o, bb.e16 + o, bb.dg + (int64_t)z * bb.mp, bb.mp, g.first ? bb.scale[2 * z + 1] : 1.f};
  }
  static __device__ float prescale(const Ctx& x) { return x.pre; }
  static __device__ int views(const Ctx&, bool diag) { return diag ? kViewRow : kViewRow | kViewCol; }
  // The transposed tile of E comes from LDS; A itself is stored only for
  // the tiles this phase computes (one side of the diagonal), the only ones
  // the polynomial reads.
  static constexpr bool kMirror = true;
  static constexpr bool kLower = true;
  static constexpr bool kAddX = false;
  struct Aux {};
  static constexpr int kBatch = 32, kBatchLast = 0;
  static constexpr bool kFastPath = false;
  template <bool>
  static __device__ Aux load(const Ctx&, int, int, int) { return Aux{}; }
  static __device__ void store_t(const Ctx& x, int r, int c, u32x4_t v) {
    *reinterpret_cast<MUON_GLOBAL u32x4_t*>(as_global(x.e16 + (int64_t)r * x.mp + c)) = v;
  }
  template <bool>
  static __device__ f32x4_t store(const Ctx& x, int, int r, int c, f32x4_t v, Aux) {
    const int64_t idx = (int64_t)r * x.mp + c;
    st_f32x4(x.a32 + idx, v);
    const int d = r - c;  // position of the diagonal in this piece, if any
    if (d >= 0 && d < 4) {
      const float dv = d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
      *reinterpret_cast<MUON_GLOBAL float*>(as_global(x.dg + r)) = dv;
      v.x = d == 0 ? 0.f : v.x;
      v.y = d == 1 ? 0.f : v.y;
      v.z = d == 2 ? 0.f : v.z;
      v.w = d == 3 ? 0.f : v.w;
    }
    st_bf16x4(x.e16 + idx, v);
    return v;
  }
};

// R = (a - 1) I + b A + c (E E + diag(d) A + A diag(d) - diag(d)^2), in bf16.
struct PolyPhase {
  static __device__ Operands operands(const BigArgs&, const BigBucket& bb, int z) {
    const char* e = reinterpret_cast<const char*>(bb.e16 + (int64_t)z * bb.mp * bb.mp);
    return Operands{e, e, bb.mp, bb.mp, big_k_over_m(bb.m)};
  }
  struct Ctx {
    const float* a32;
    const float* dg;
    uint16_t* r16;
    int64_t mp;
    float b, c, am1;
  };
  static __device__ Ctx context(const BigArgs& g, const BigBucket& bb, int z) {
    const int64_t o = (int64_t)z * bb.mp * bb.mp;
    return Ctx{bb.a32 + o, bb.dg + (int64_t)z * bb.mp, bb.r16 + o, bb.mp, g.sc->b, g.sc->c, g.sc->a - 1.f};
  }
  static __device__ float prescale(const Ctx&) { return 1.f; }
  static __device__ int views(const Ctx&, bool diag) { return diag ? kViewRow : kViewRow | kViewCol; }
  // R is symmetric: its transposed tile comes from LDS, so A is read only
  // for the tiles the Gram phase computed (the same side of the diagonal).
  static constexpr bool kMirror = true;
  static constexpr bool kLower = true;
  static constexpr bool kAddX = false;
  static __device__ void store_t(const Ctx& x, int r, int c, u32x4_t v) {
    *reinterpret_cast<MUON_GLOBAL u32x4_t*>(as_global(x.r16 + (int64_t)r * x.mp + c)) = v;
  }
  struct Aux {
    f32x4_t a, dc;  // A (r, c .. c+3) and d (c .. c+3)
    float dr;       // d (r)
  };
  static constexpr int kBatch = 4, kBatchLast = 16;
  static constexpr bool kFastPath = false;
  template <bool>
  static __device__ Aux load(const Ctx& x, int, int r, int c) {
    return Aux{ld_f32x4(x.a32 + (int64_t)r * x.mp + c), ld_f32x4(x.dg + c),
               *reinterpret_cast<const MUON_GLOBAL float*>(as_global(x.dg + r))};
  }
  template <bool>
  static __device__ f32x4_t store(const Ctx& x, int, int r, int c, f32x4_t ee, const Aux& q) {
    const int64_t idx = (int64_t)r * x.mp + c;
    const f32x4_t a = q.a, dc = q.dc;
    const float dr = q.dr;
    f32x4_t o;
#define MUON_POLY_ONE(comp, u)                                                      \
    {                                                                               \
      const bool on_diag = r == c + (u);                                            \
      const float a2 = ee.comp + (on_diag ? dr * dr : (dr + dc.comp) * a.comp);     \
      o.comp = x.b * a.comp + x.c * a2 + (on_diag ? x.am1 : 0.f);                   \
    }
    MUON_POLY_ONE(x, 0)
    MUON_POLY_ONE(y, 1)
    MUON_POLY_ONE(z, 2)
    MUON_POLY_ONE(w, 3)
#undef MUON_POLY_ONE
    st_bf16x4(x.r16 + idx, o);
    return o;
  }
};

// Operands of R X: rows of R and rows of X^T (both contiguous along k = m).
// The X term of X + R X is added to the accumulators from the X^T slices in
// LDS (kAddX), so neither epilogue reads X.
__device__ __forceinline__ Operands apply_operands(const BigArgs& g, const BigBucket& bb, int z) {
  return Operands{reinterpret_cast<const char*>(bb.r16 + (int64_t)z * bb.mp * bb.mp),
                  bb.xt[g.src] + (int64_t)z * bb.np * bb.mp * 2, bb.mp, bb.mp, big_k_over_m(bb.m)};
}

// X' = s (X + R X): X' [mp][np] from the row view, X'^T [np][mp] written
// from LDS (the same values).
struct ApplyPhase {
  static __device__ Operands operands(const BigArgs& g, const BigBucket& bb, int z) {
    return apply_operands(g, bb, z);
  }
  struct Ctx {
    uint16_t* x_new;
    uint16_t* xt_new;
    int64_t mp, np;
    float pre;
  };
  static __device__ Ctx context(const BigArgs& g, const BigBucket& bb, int z) {
    const int64_t o = (int64_t)z * bb.mp * bb.np * 2;
    return Ctx{reinterpret_cast<uint16_t*>(bb.x[g.src ^ 1] + o), reinterpret_cast<uint16_t*>(bb.xt[g.src ^ 1] + o),
               bb.mp, bb.np, g.first ? bb.scale[2 * z] : 1.f};
  }
  static __device__ float prescale(const Ctx& x) { return x.pre; }
  static __device__ int views(const Ctx&, bool) { return kViewRow | kViewCol; }
  static constexpr bool kMirror = true;
  static constexpr bool kLower = false;
  static constexpr bool kAddX = true;
  struct Aux {};
  static constexpr int kBatch = 32, kBatchLast = 0;
  static constexpr bool kFastPath = false;
  template <bool>
  static __device__ Aux load(const Ctx&, int, int, int) { return Aux{}; }
  template <bool>
  static __device__ f32x4_t store(const Ctx& x, int, int r, int c, f32x4_t v, Aux) {
    st_bf16x4(x.x_new + (int64_t)r * x.np + c, v);
    return v;
  }
  static __device__ void store_t(const Ctx& x, int r, int c, u32x4_t v) {
    *reinterpret_cast<MUON_GLOBAL u32x4_t*>(as_global(x.xt_new + (int64_t)r * x.mp + c)) = v;
  }
};

// Last round: W <- W - decay W - lr f s (X + R X) through the slice's own
// layout (the row view for a slice stored [m, n], the column view for one
// stored [n, m]); decay = lr wd and f the shape factor (both options).
struct FinalPhase {
  static __device__ Operands operands(const BigArgs& g, const BigBucket& bb, int z) {
    return apply_operands(g, bb, z);
  }
  struct Ctx {
    char* w;
    int64_t rows, len;   // stored rows and row length of the slice
    int pdtype, view, vec;
    float k;             // lr f s
    float decay;         // lr wd
  };
  static __device__ Ctx context(const BigArgs& g, const BigBucket& bb, int z) {
    const DevMat d = bb.mats[z];
    const PtrEntry pe = g.ptrs[d.param];
    Ctx x;
    x.w = static_cast<char*>(pe.w) + d.slice_off * (d.pdtype == 1 ? 2 : 4);
    x.view = d.transposed ? kViewCol : kViewRow;
    x.rows = d.transposed ? bb.n : bb.m;
    x.len = d.transposed ? bb.m : bb.n;
    x.pdtype = d.pdtype;
    x.vec = bb.vec;
    x.k = g.sc->lr * update_factor(g.sc->scale_mode, bb.m, bb.n, d.transposed) * (g.first ? bb.scale[2 * z] : 1.f);
    x.decay = g.sc->decay;
    return x;
  }
  static __device__ float prescale(const Ctx&) { return 1.f; }
  static __device__ int views(const Ctx& x, bool) { return x.view; }
  static constexpr bool kMirror = false;
  static constexpr bool kLower = false;
  static constexpr bool kAddX = true;
  static __device__ void store_t(const Ctx&, int, int, u32x4_t) {}  // no transposed copy
  struct Aux {
    f32x4_t w;   // W (r, c .. c+3) as float32 (entries past the row end unused)
  };
  static constexpr int kBatch = 4, kBatchLast = 16;
  // The unguarded path: a float32 W whose rows are whole 16-byte groups, and
  // an epilogue pass (128 rows of a tile) that lies wholly inside the slice
  // (every tile of a slice whose sides are multiples of 256).
  static constexpr bool kFastPath = true;
  static __device__ bool fast(const Ctx& x, int, int row0, int col0) {
    return x.vec && x.pdtype == 0 && row0 + 128 <= x.rows && col0 + kBigTile <= x.len;
  }
  template <bool kUnguarded>
  static __device__ Aux load(const Ctx& x, int, int r, int c) {
    Aux q{};
    if constexpr (kUnguarded) {
      q.w = *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(x.w) + 4 * ((int64_t)r * x.len + c));
      return q;
    }
    if (r >= x.rows || c >= x.len) return q;
    const int64_t idx = (int64_t)r * x.len + c;
    if (x.vec && c + 3 < x.len) {
      if (x.pdtype == 1) {  // bfloat16 W
        const u32x2_t w = *reinterpret_cast<const MUON_GLOBAL u32x2_t*>(as_global(x.w) + 2 * idx);
        q.w = f32x4_t{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
      } else {
        q.w = *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(x.w) + 4 * idx);
      }
    } else {
      q.w.x = load_as_f32(x.w, idx, x.pdtype);
      q.w.y = c + 1 < x.len ? load_as_f32(x.w, idx + 1, x.pdtype) : 0.f;
      q.w.z = c + 2 < x.len ? load_as_f32(x.w, idx + 2, x.pdtype) : 0.f;
      q.w.w = c + 3 < x.len ? load_as_f32(x.w, idx + 3, x.pdtype) : 0.f;
    }
    return q;
  }
  template <bool kUnguarded>
  static __device__ f32x4_t store(const Ctx& x, int, int r, int c, f32x4_t v, const Aux& q) {
    const f32x4_t n{q.w.x - x.decay * q.w.x - x.k * v.x, q.w.y - x.decay * q.w.y - x.k * v.y,
                    q.w.z - x.decay * q.w.z - x.k * v.z, q.w.w - x.decay * q.w.w - x.k * v.w};
    const int64_t idx = (int64_t)r * x.len + c;
    if constexpr (kUnguarded) {
      *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(x.w) + 4 * idx) = n;
      return n;
    }
    if (r >= x.rows || c >= x.len) return v;
    if (x.vec && c + 3 < x.len) {
      if (x.pdtype == 1) {  // bfloat16 W, rounded to nearest even
        *reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(x.w) + 2 * idx) =
            u32x2_t{pack_bf16x2(n.x, n.y), pack_bf16x2(n.z, n.w)};
      } else {
        *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(x.w) + 4 * idx) = n;
      }
      return n;
    }
    store_from_f32(x.w, idx, x.pdtype, n.x);
    if (c + 1 < x.len) store_from_f32(x.w, idx + 1, x.pdtype, n.y);
    if (c + 2 < x.len) store_from_f32(x.w, idx + 2, x.pdtype, n.z);
    if (c + 3 < x.len) store_from_f32(x.w, idx + 3, x.pdtype, n.w);
    return n;
  }
};

}  // namespace

hipError_t launch_big(BigKind kind, const BigArgs& a, hipStream_t s) {
  const dim3 grid(a.t8), block(kThreadsBig);
  switch (kind) {
    case kBigGram: hipLaunchKernelGGL(k_gemm_big<GramPhase>, grid, block, 0, s, a); break;
    case kBigPoly: hipLaunchKernelGGL(k_gemm_big<PolyPhase>, grid, block, 0, s, a); break;
    case kBigApply: hipLaunchKernelGGL(k_gemm_big<ApplyPhase>, grid, block, 0, s, a); break;
    case kBigFinal: hipLaunchKernelGGL(k_gemm_big<FinalPhase>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace muon
