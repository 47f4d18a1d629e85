// layout.h -- plain structures shared by the host planner and the kernels.
//
// No HIP types here: the planner is pure host code that also runs where no
// GPU exists (muon_plan_describe).
#pragma once
#include <stdint.h>

namespace muon {

constexpr int kMaxResidentM = 32;     // resident path: one 32-row MFMA tile holds all of m
constexpr int kResidentWaves = 8;     // waves per resident workgroup (512 threads)
constexpr int kStreamPad = 128;       // streamed workspace dims are padded to this
constexpr int kMomTile = 64;          // momentum kernel tile (oriented 64 x 64)

enum KernelClass { kClsResident = 0, kClsMomentum, kClsNorm, kClsGram, kClsPoly, kClsApply,
                   kClsUpdate, kNumClasses };

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
