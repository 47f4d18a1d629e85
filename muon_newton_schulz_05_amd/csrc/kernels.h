// kernels.h -- host-side launchers of the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/muon.h"
#include "layout.h"

namespace muon {

// Writes the step's scalars.
hipError_t launch_prologue(DevScalars* dst, const DevScalars& v, hipStream_t s);

// ---------------------------------------------------------------- fixed scratch (muon_step_noalloc)
constexpr uint64_t kScratchBytes = MUON_NOALLOC_SCRATCH_BYTES;
// Device address of the fixed scratch array on `device` (looked up once per
// device, then cached).
hipError_t scratch_address(int device, char** out);
// Zero `bytes` (a multiple of 16) at p with a kernel on s.
hipError_t launch_fill_zero(void* p, uint64_t bytes, hipStream_t s);

// ---------------------------------------------------------------- skinny (m <= 32)
// The first kernel of an eager step carries the step's scalars by value and
// writes them to the plan's scalar block for the kernels after it (sc_out
// non-null); every other launch reads them from the block (sc).
struct SkinnyLaunch {
  SkinnyBucket b0;                // the first skinny bucket, by value
  const SkinnyBucket* buckets;    // every skinny bucket of the plan (device table)
  int n_buckets;
  const PtrEntry* ptrs;
  const DevScalars* sc;
  DevScalars sv;          // scalars by value (used when sc_out is set)
  DevScalars* sc_out;     // null, or the scalar block to fill
  uint32_t* err;          // device error word
  int items;              // (slice, chunk) items over all buckets
  int slices;             // slices over all buckets
  int m_max;              // largest m (sizes LDS; the polynomial's k steps)
  int bf16;               // 1: bf16 matrix-core mode, 0: fp32 mode
  int nesterov;           // the plan's Nesterov option (selects the apply kernel)
};
hipError_t launch_skinny_gram(const SkinnyLaunch& a, hipStream_t s);
hipError_t launch_skinny_poly(const SkinnyLaunch& a, hipStream_t s);
hipError_t launch_skinny_apply(const SkinnyLaunch& a, hipStream_t s);

// ---------------------------------------------------------------- streamed
struct MomentumLaunch {
  const DevMat* mats;
  const PtrEntry* ptrs;
  const DevScalars* sc;
  DevScalars sv;          // as in SkinnyLaunch
  DevScalars* sc_out;
  void* x;                // [count][mp][np]
  void* xt;               // [count][np][mp]
  float* sq;              // [count][km_tiles]
  int64_t m, n, mp, np;
  int count, km_tiles, x_bytes;
};
hipError_t launch_momentum(const MomentumLaunch& a, hipStream_t s);

struct NormLaunch {
  const float* sq;
  float* scale;           // [count][2] = {s, s*s}
  const DevScalars* sc;
  uint32_t* err;          // device error word: kErrNonFinite when a sum is not finite
  int count, km_tiles;
};
hipError_t launch_norm(const NormLaunch& a, hipStream_t s);

// ---------------------------------------------------------------- streamed products (grouped)
// One launch per product phase covers every bucket of a group: the small
// buckets (padded m <= kSmallMaxMp: 32 x 32 output tiles, the contraction
// split over 4 waves), or the other streamed buckets that do not take the
// large tiles (BT x BT output tiles).  Both read this bucket array.
struct SmallArgs {
  const SmallBucket* buckets;
  int nb;
  int src;                // this round reads X[src], X^T[src]
  int first;              // first round: fold the normalisation scale in
  const DevScalars* sc;
  const PtrEntry* ptrs;
};
// phase 0 gram, 1 poly, 2 apply (final_round: W update); f32_operands: fp32
// mode (else bf16 X and a bf16 hi/lo P).  wgs: workgroups of the phase.
hipError_t launch_small(int phase, bool final_round, bool f32_operands, const SmallArgs& a, int64_t wgs,
                        hipStream_t s);
// The same for the other group; bt: the output tile (64 or 128) of this
// phase, in whose units the buckets' t0 and wgs count.
hipError_t launch_mid(int phase, bool final_round, bool f32_operands, const SmallArgs& a, int64_t wgs, int bt,
                      hipStream_t s);

// ---------------------------------------------------------------- streamed, large bf16 buckets
// One launch per product phase covers every large bucket; the tile table
// (entries: bucket, slice, 256 x 256 output tile) fixes the order.
enum BigKind { kBigGram = 0, kBigPoly = 1, kBigApply = 2, kBigFinal = 3 };
struct BigArgs {
  const BigBucket* buckets;
  const BigTile* tiles;
  int t8;                 // table length (multiple of 8)
  int src;                // this round reads X[src], X^T[src]
  int first;              // first round: fold the normalisation scale in
  const DevScalars* sc;
  const PtrEntry* ptrs;
};
//  kBigGram   A = s2 X X^T -> a32, dg = diag(A), e16 = A - diag(A) (bf16)
//  kBigPoly   R = (a - 1) I + b A + c (E E + diag(d) A + A diag(d) - diag(d)^2) -> r16
//  kBigApply  X'[src^1] = s (X + R X), with X'^T alongside
//  kBigFinal  W <- W - lr s (X + R X) through each slice's storage layout
hipError_t launch_big(BigKind kind, const BigArgs& a, hipStream_t s);

// ns_steps == 0: W -= lr * s * M.
struct Update0Launch {
  const DevMat* mats;
  const PtrEntry* ptrs;
  const DevScalars* sc;
  const float* scale;
  int64_t m, n;
  int count;
};
hipError_t launch_update0(const Update0Launch& a, hipStream_t s);

}  // namespace muon
