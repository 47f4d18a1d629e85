// layout.h -- plain structures shared by the host planner and the kernels.
//
// No HIP types here: the planner is pure host code that also runs where no
// GPU exists (muon_plan_describe).
#pragma once
#include <stdint.h>

namespace muon {

constexpr int kMaxSkinnyM = 32;       // skinny path: one 32-row MFMA tile holds all of m
constexpr int kSkinnyChunk = 256;     // skinny path: columns per workgroup (fixed by n alone)
constexpr int kStreamPad = 128;       // streamed workspace dims are padded to this
constexpr int kBigTile = 256;         // large bf16 buckets: product tile, and their padding
constexpr int kBigMinM = 513;         // bf16 buckets with m >= this take the large-tile products
constexpr uint32_t kNoTile = 0xFFFFFFFFu;  // tile-table padding entry
constexpr int kMomTile = 64;          // momentum kernel tile (oriented 64 x 64)

enum KernelClass { kClsSkinnyGram = 0, kClsSkinnyPoly, kClsSkinnyApply, kClsMomentum, kClsNorm,
                   kClsGram, kClsPoly, kClsApply, kClsUpdate, kNumClasses };

// Bits of the plan's device error word.
constexpr uint32_t kErrNonFinite = 1u;  // a slice's momentum norm was not finite

// Scalars of one step, written to device memory by the prologue kernel.
struct DevScalars {
  float lr, beta, a, b, c, eps;
  int32_t ns_steps;
  int32_t pad;
};

// Device pointers of one parameter.
struct PtrEntry {
  void* w;
  const void* g;
  float* m;
};

// One 2-D slice as the kernels see it.
struct DevMat {
  int32_t param;       // row of the pointer table
  int32_t transposed;  // stored as [n, m] (R > C)
  int32_t pdtype;      // muon_dtype_t of W
  int32_t gdtype;      // muon_dtype_t of G
  int64_t slice_off;   // element offset of the slice inside its parameter
};

}  // namespace muon
