// planner.h -- host-side planning of a fused Muon step (no HIP calls).
//
// Groups 2-D slices by oriented shape so that each group runs as one batched
// problem ("MindSpore HyperParallel X 盘古,Muon优化器实现6倍性能跃升", section
// 矩阵融合优化 / matrix fusion: parameters whose last two dimensions agree are
// stacked into one [B, M, N] problem; section 专家切分 / expert split: each
// slice of a 3-D expert tensor is independent), picks a kernel path per group
// and lays out the device workspace.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/muon.h"
#include "layout.h"

namespace muon {

struct Slice {
  int param = 0, e = 0, transposed = 0, pdtype = 0, gdtype = 0;
  int64_t rows = 0, cols = 0, m = 0, n = 0, slice_off = 0;
  int bucket = -1;
};

// Slices per bucket: the launches index them in a grid dimension.
constexpr int64_t kMaxBucketSlices = 65535;

struct BucketPlan {
  int64_t m = 0, n = 0;
  int path = MUON_PATH_STREAM;
  std::vector<int> slices;  // indices into Plan::slices, in plan order
  int n_transposed = 0;

  // skinny path (m <= 32)
  int n_chunks = 0;         // 256-column chunks per slice
  uint64_t off_gram = 0, off_qs = 0;

  // streamed path
  bool big = false;         // bf16 mode and m >= the plan's large_min_m: 256 x 256 tile products
  bool small = false;       // padded m <= kSmallMaxMp: grouped 32 x 32 tile products
  int64_t mp = 0, np = 0;   // padded dims
  int x_bytes = 0;          // X element size (2: bf16, 4: fp32)
  bool poly_f32 = false;    // A^2 from float32 A (else bf16 copy of A)
  bool p_hilo = false;      // B fed to the matrix cores as a bf16 hi/lo pair
  int km_tiles = 0;         // momentum-kernel tiles per slice
  uint64_t off_x[2] = {0, 0}, off_xt[2] = {0, 0};
  uint64_t off_a32 = 0, off_a16 = 0, off_phi = 0, off_plo = 0, off_sq = 0, off_scale = 0;
  uint64_t off_dg = 0;      // big: diagonal of A per slice

  uint64_t off_mats = 0;    // this bucket's DevMat table
  uint64_t ws_begin = 0, ws_bytes = 0;
};

struct Plan {
  int mode = MUON_MODE_BF16_MFMA;
  float eps = 1e-7f;
  int max_ns_steps = 16;
  uint64_t workspace_limit = 0;
  int skinny_max_m = kMaxSkinnyM;
  int64_t large_min_m = kBigMinM;  // bf16 mode: m from which slices take the large tiles
  int timing = 0, use_graph = 0;
  int nesterov = 0, update_scale = MUON_SCALE_NONE;  // update variants
  float weight_decay = 0.f;
  int n_cu = 256;

  int n_params = 0;
  std::vector<muon_param_desc_t> descs;
  std::vector<Slice> slices;
  std::vector<BucketPlan> buckets;
  uint64_t off_scalars = 0, off_err = 0, off_ptrs = 0;
  // Large bf16 buckets: their indices, the device BigBucket array and one
  // tile table per product phase (kBigGram, kBigPoly, kBigApply).
  std::vector<int> big;
  uint64_t off_big_params = 0;
  // Skinny buckets: their indices, the device SkinnyBucket array and the
  // totals of the grouped launches.
  std::vector<int> skinny;
  uint64_t off_skinny_params = 0;
  int skinny_items = 0, skinny_slices = 0, skinny_m_max = 0;
  std::vector<BigTile> big_tab[3];
  uint64_t off_big_tab[3] = {0, 0, 0};
  // Small streamed buckets: their indices, the device SmallBucket array and
  // the workgroups of each grouped phase launch (gram, poly, apply).
  std::vector<int> small;
  uint64_t off_small_params = 0;
  int64_t small_wgs[3] = {0, 0, 0};
  // The other streamed buckets (not skinny, small or large): their indices,
  // the device SmallBucket array, and per product phase the output tile
  // (128, or 64 when the group has fewer 128-tiles than kMidMinTiles) and
  // the workgroups in those tiles.
  std::vector<int> mid;
  uint64_t off_mid_params = 0;
  int mid_bt[3] = {128, 128, 128};
  int64_t mid_wgs[3] = {0, 0, 0};
  uint64_t ws_total = 0;
  int launches_fixed = 0, launches_per_ns = 0;
};

void default_opts(muon_plan_opts_t* o);

// Validate and plan.  n_cu describes the device (create) or the assumed
// device (describe).  Returns a muon_status_t; *err gets a message.
int make_plan(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts,
              int n_cu, Plan* out, std::string* err);

void fill_info(const Plan& p, muon_plan_info_t* info);

// Tile table of one product phase over the plan's large buckets (phase 0:
// X X^T, 1: E E, 2: R X).  Output tiles are grouped in blocks of 4 tile rows
// x 8 tile columns of one slice (for the symmetric phases only tiles on or
// above the diagonal, with the 8 x 8 triangles on the diagonal as blocks of
// their own); blocks are dealt, longest contraction first, to the 8 XCD
// stretches of the table, each block to the stretch with the least work so
// far; stretches are padded with kNoTile to a common length.
std::vector<BigTile> big_table(const Plan& p, int phase);

}  // namespace muon
