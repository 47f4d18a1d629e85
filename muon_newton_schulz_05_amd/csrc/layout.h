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
constexpr int kBigMinM = 129;         // default: bf16 buckets with m >= this take the large-tile products
constexpr int kBigKStep = 64;         // large-tile products: k elements per slice
// Longest padded n of the large-tile products: 255 rows of n bf16 plus a
// 16-byte chunk offset stay below 2^32 bytes.
constexpr int64_t kBigMaxN = int64_t(1) << 23;
// Contraction length of the large-tile products over a dimension of d (m, or
// n for the Gram): operand entries past d are zero, so the k loop stops at d
// rounded up to a slice.
inline constexpr int64_t big_k_over_m(int64_t d) { return (d + kBigKStep - 1) / kBigKStep * kBigKStep; }
constexpr uint32_t kNoTile = 0xFFFFFFFFu;  // tile-table padding entry
constexpr int kMomTile = 64;          // momentum kernel tile (oriented 64 x 64)
constexpr int kSmallMaxMp = 256;      // streamed buckets with padded m <= this: grouped 32 x 32 products
constexpr int kSmallTile = 32;        // their output tile
constexpr int kMidMinTiles = 256;     // other streamed buckets: fewer 128-tiles per phase than this take 64-tiles

enum KernelClass { kClsSkinnyGram = 0, kClsSkinnyPoly, kClsSkinnyApply, kClsMomentum, kClsNorm,
                   kClsGram, kClsPoly, kClsApply, kClsUpdate, kNumClasses };

// Bits of the plan's device error word.
constexpr uint32_t kErrNonFinite = 1u;  // a slice's momentum norm was not finite

// Scalars of one step (carried by value to the step's first kernel, which
// writes them to the plan's scalar block; or written by a prologue kernel).
struct DevScalars {
  float lr, beta, a, b, c, eps;
  float decay;          // lr * weight decay: W <- W - decay W - lr f O
  int32_t ns_steps;
  int32_t nesterov;     // orthogonalise G + beta M instead of M
  int32_t scale_mode;   // muon_update_scale_t
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

// One skinny bucket as the kernels see it.  The skinny stages run as one
// launch each over all skinny buckets; a workgroup finds its bucket in a
// device array of these by its first item or slice (the first bucket also
// rides in the launch arguments).
struct SkinnyBucket {
  const DevMat* mats;  // slice table
  double* gram_parts;  // [count][n_chunks][m(m+1)/2]: upper triangles, packed by rows
  float* qs;           // [count][32*32]: s * Q
  int32_t m, n, n_chunks, count;
  int32_t item0;       // first (slice, chunk) item of the Gram and apply launches
  int32_t slice0;      // first slice of the polynomial launch
};

// Large bf16 buckets run each product phase as one launch over all of
// them: a tile table entry names the bucket, the slice and the output tile.
struct BigTile {
  uint32_t bz;  // bucket << 24 | slice; kNoTile marks padding
  uint32_t mn;  // tm | tn << 16 (256 x 256 output tiles)
};

// Device addresses of one streamed bucket that does not take the large tiles
// (the small ones, padded m <= kSmallMaxMp, form one group, the others
// another).  Each product phase of a round is one launch over a group;
// workgroup b belongs to the last bucket with t0[phase] <= b.
struct SmallBucket {
  const DevMat* mats;  // slice table
  char* x[2];          // X ping-pong, [count][mp][np] (bf16 or float)
  char* xt[2];         // X^T ping-pong, [count][np][mp]
  float* a32;          // A, [count][mp][mp]
  char* phi;           // P (float), or its bf16 high part
  uint16_t* plo;       // bf16 low part of P (bf16 mode), else null
  float* scale;        // [count][2] = {s, s^2}
  int64_t m, n, mp, np;
  int32_t count;
  int32_t t0[3];       // first workgroup of the bucket in the gram, poly and apply launches
};

// Device addresses of one large bucket's workspace (filled at plan creation).
struct BigBucket {
  char* x[2];          // X ping-pong, [count][mp][np] bf16
  char* xt[2];         // X^T ping-pong, [count][np][mp] bf16
  float* a32;          // A, [count][mp][mp]
  uint16_t* e16;       // A without its diagonal, bf16
  float* dg;           // diagonal of A, [count][mp]
  uint16_t* r16;       // (a - 1) I + b A + c A^2, bf16
  float* scale;        // [count][2] = {s, s^2}
  const DevMat* mats;  // slice table
  int64_t m, n, mp, np;
  int32_t vec;         // m and n are multiples of 4 (whole 16-byte W groups)
  int32_t pad;
};

}  // namespace muon
