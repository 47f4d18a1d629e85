// planner.cpp -- validation, orientation, shape buckets and workspace layout.
#include "planner.h"

#include <algorithm>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <utility>

namespace muon {

namespace {

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Alloc {
  uint64_t top = 0;
  uint64_t take(uint64_t bytes) {
    uint64_t off = align_up(top, 256);
    top = off + bytes;
    return off;
  }
};

}  // namespace

void default_opts(muon_plan_opts_t* o) {
  std::memset(o, 0, sizeof(*o));
  o->mode = MUON_MODE_BF16_MFMA;
  o->use_graph = 0;
  o->eps = 1e-7f;
  o->max_ns_steps = 16;
  o->workspace_limit = 0;
  o->skinny_max_m = 0;
  o->large_min_m = 0;
  o->timing = 0;
  o->n_cu = 0;
}

int make_plan(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts_in,
              int n_cu, Plan* out, std::string* err) {
  char buf[256];
  if (descs == nullptr || out == nullptr) {
    *err = "null descriptor array or output";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (n_params <= 0) {
    *err = "n_params must be positive";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  muon_plan_opts_t opts;
  if (opts_in) opts = *opts_in;
  else default_opts(&opts);
  if (opts.mode != MUON_MODE_FP32 && opts.mode != MUON_MODE_BF16_MFMA) {
    *err = "unknown mode";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(opts.eps) || opts.eps < 0.f) {
    *err = "eps must be finite and >= 0";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (opts.max_ns_steps < 0 || opts.max_ns_steps > 1000) {
    *err = "max_ns_steps must be in [0, 1000]";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (opts.skinny_max_m < -1 || opts.skinny_max_m > kMaxSkinnyM) {
    std::snprintf(buf, sizeof buf, "skinny_max_m must be -1, 0 or in [1, %d]", kMaxSkinnyM);
    *err = buf;
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (opts.large_min_m < -1 || (opts.large_min_m > 0 && opts.large_min_m <= kMaxSkinnyM)) {
    std::snprintf(buf, sizeof buf, "large_min_m must be -1, 0 or at least %d", kMaxSkinnyM + 1);
    *err = buf;
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (opts.nesterov != 0 && opts.nesterov != 1) {
    *err = "nesterov must be 0 or 1";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (opts.update_scale < MUON_SCALE_NONE || opts.update_scale > MUON_SCALE_RMS) {
    *err = "unknown update_scale";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(opts.weight_decay) || opts.weight_decay < 0.f) {
    *err = "weight_decay must be finite and >= 0";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (n_cu <= 0) {
    *err = "device description has no compute units";
    return MUON_ERR_INVALID_ARGUMENT;
  }

  Plan p;
  p.mode = opts.mode;
  p.eps = opts.eps;
  p.max_ns_steps = opts.max_ns_steps;
  p.workspace_limit = opts.workspace_limit;
  p.skinny_max_m = opts.skinny_max_m == 0 ? kMaxSkinnyM
                   : opts.skinny_max_m < 0 ? 0 : opts.skinny_max_m;
  p.large_min_m = opts.large_min_m == 0 ? kBigMinM
                  : opts.large_min_m < 0 ? INT32_MAX : opts.large_min_m;
  p.timing = opts.timing ? 1 : 0;
  p.use_graph = opts.use_graph ? 1 : 0;
  p.nesterov = opts.nesterov;
  p.update_scale = opts.update_scale;
  p.weight_decay = opts.weight_decay;
  p.n_cu = n_cu;
  p.n_params = n_params;
  p.descs.assign(descs, descs + n_params);

  // Expand parameters into 2-D slices and orient each one.
  for (int i = 0; i < n_params; ++i) {
    const muon_param_desc_t& d = descs[i];
    if (d.ndim != 2 && d.ndim != 3) {
      std::snprintf(buf, sizeof buf, "parameter %d: ndim %d (Muon takes 2-D matrices or 3-D stacks)",
                    i, d.ndim);
      *err = buf;
      return MUON_ERR_INVALID_ARGUMENT;
    }
    for (int k = 0; k < d.ndim; ++k) {
      if (d.shape[k] <= 0 || d.shape[k] >= (int64_t(1) << 31)) {
        std::snprintf(buf, sizeof buf, "parameter %d: dimension %d is %lld", i, k,
                      (long long)d.shape[k]);
        *err = buf;
        return MUON_ERR_INVALID_ARGUMENT;
      }
    }
    if ((d.param_dtype != MUON_F32 && d.param_dtype != MUON_BF16) ||
        (d.grad_dtype != MUON_F32 && d.grad_dtype != MUON_BF16)) {
      std::snprintf(buf, sizeof buf, "parameter %d: unknown dtype", i);
      *err = buf;
      return MUON_ERR_INVALID_ARGUMENT;
    }
    const int64_t E = d.ndim == 3 ? d.shape[0] : 1;
    const int64_t R = d.shape[d.ndim - 2], C = d.shape[d.ndim - 1];
    if (E * R * C >= (int64_t(1) << 40)) {
      std::snprintf(buf, sizeof buf, "parameter %d: too many elements", i);
      *err = buf;
      return MUON_ERR_INVALID_ARGUMENT;
    }
    for (int64_t e = 0; e < E; ++e) {
      Slice s;
      s.param = i;
      s.e = (int)e;
      s.rows = R;
      s.cols = C;
      s.transposed = R > C ? 1 : 0;
      s.m = s.transposed ? C : R;
      s.n = s.transposed ? R : C;
      s.slice_off = e * R * C;
      s.pdtype = d.param_dtype;
      s.gdtype = d.grad_dtype;
      p.slices.push_back(s);
    }
  }

  // Bucket by oriented shape, in order of first appearance.  Launches put
  // the slice index of a bucket in a grid dimension that holds at most
  // kMaxBucketSlices, so a larger group of one shape fills several buckets.
  std::map<std::pair<int64_t, int64_t>, int> index;
  for (int si = 0; si < (int)p.slices.size(); ++si) {
    Slice& s = p.slices[si];
    auto key = std::make_pair(s.m, s.n);
    auto it = index.find(key);
    int b;
    if (it == index.end() || (int64_t)p.buckets[it->second].slices.size() >= kMaxBucketSlices) {
      if ((int)p.buckets.size() >= MUON_MAX_BUCKETS) {
        std::snprintf(buf, sizeof buf, "more than %d distinct oriented shapes", MUON_MAX_BUCKETS);
        *err = buf;
        return MUON_ERR_UNSUPPORTED;
      }
      b = (int)p.buckets.size();
      index[key] = b;
      BucketPlan bp;
      bp.m = s.m;
      bp.n = s.n;
      bp.path = s.m <= p.skinny_max_m ? MUON_PATH_SKINNY : MUON_PATH_STREAM;
      p.buckets.push_back(bp);
    } else {
      b = it->second;
    }
    s.bucket = b;
    p.buckets[b].slices.push_back(si);
    p.buckets[b].n_transposed += s.transposed;
  }

  // Geometry and workspace.
  Alloc ws;
  p.off_scalars = ws.take(sizeof(DevScalars));
  p.off_err = ws.take(sizeof(uint32_t));
  p.off_ptrs = ws.take(sizeof(PtrEntry) * (uint64_t)n_params);
  p.launches_fixed = p.use_graph ? 1 : 0;  // graph replays need a prologue kernel for the scalars
  p.launches_per_ns = 0;
  for (BucketPlan& bp : p.buckets) {
    const uint64_t cnt = bp.slices.size();
    bp.ws_begin = ws.take(0);
    bp.off_mats = ws.take(sizeof(DevMat) * cnt);
    if (bp.path == MUON_PATH_SKINNY) {
      bp.n_chunks = (int)((bp.n + kSkinnyChunk - 1) / kSkinnyChunk);
      bp.off_gram = ws.take(cnt * bp.n_chunks * (bp.m * (bp.m + 1) / 2) * sizeof(double));  // upper triangles
      bp.off_qs = ws.take(cnt * 1024 * sizeof(float));
    } else {
      // The large-tile products address a 256-row operand panel with 32-bit
      // lane offsets and a tile column in 16 bits, so slices longer than
      // kBigMaxN take the general products instead.
      bp.big = p.mode == MUON_MODE_BF16_MFMA && bp.m >= p.large_min_m && round_up(bp.n, kBigTile) <= kBigMaxN;
      const int64_t pad = bp.big ? kBigTile : kStreamPad;
      bp.mp = round_up(bp.m, pad);
      bp.np = round_up(bp.n, pad);
      bp.x_bytes = p.mode == MUON_MODE_FP32 ? 4 : 2;
      bp.poly_f32 = !bp.big;
      bp.p_hilo = p.mode == MUON_MODE_BF16_MFMA && !bp.big;
      bp.km_tiles = (int)(((bp.m + kMomTile - 1) / kMomTile) * ((bp.n + kMomTile - 1) / kMomTile));
      const uint64_t xsz = cnt * bp.mp * bp.np * bp.x_bytes;
      const uint64_t msz = cnt * bp.mp * bp.mp;
      for (int i = 0; i < 2; ++i) bp.off_x[i] = ws.take(xsz);
      for (int i = 0; i < 2; ++i) bp.off_xt[i] = ws.take(xsz);
      bp.off_a32 = ws.take(msz * 4);
      bp.off_a16 = (p.mode == MUON_MODE_BF16_MFMA && !bp.poly_f32) ? ws.take(msz * 2) : 0;
      bp.off_phi = ws.take(msz * (p.mode == MUON_MODE_FP32 ? 4 : 2));
      bp.off_plo = bp.p_hilo ? ws.take(msz * 2) : 0;
      bp.off_sq = ws.take(cnt * bp.km_tiles * sizeof(float));
      bp.off_scale = ws.take(cnt * 2 * sizeof(float));
      if (bp.big) bp.off_dg = ws.take(cnt * bp.mp * sizeof(float));
      // Padded m <= kSmallMaxMp: 32 x 32 tile products, grouped over all such
      // buckets.  The choice depends on the shape alone, so a slice's
      // arithmetic does not depend on the plan it sits in.
      bp.small = !bp.big && bp.mp <= kSmallMaxMp;
      p.launches_fixed += 2;   // momentum, norm
    }
    bp.ws_bytes = ws.take(0) - bp.ws_begin;
  }
  // Skinny buckets share one launch per stage: momentum + Gram partials,
  // polynomial, apply + update.
  for (int b = 0; b < (int)p.buckets.size(); ++b) {
    const BucketPlan& bp = p.buckets[b];
    if (bp.path != MUON_PATH_SKINNY) continue;
    p.skinny.push_back(b);
    const int64_t items = (int64_t)p.skinny_items + (int64_t)bp.slices.size() * bp.n_chunks;
    if (items >= (int64_t(1) << 31)) {
      *err = "too many skinny column chunks in one plan";
      return MUON_ERR_UNSUPPORTED;
    }
    p.skinny_items = (int)items;
    p.skinny_slices += (int)bp.slices.size();
    p.skinny_m_max = std::max(p.skinny_m_max, (int)bp.m);
  }
  if (!p.skinny.empty()) {
    p.launches_fixed += 3;
    p.off_skinny_params = ws.take(p.skinny.size() * sizeof(SkinnyBucket));
  }
  // Small streamed buckets share one launch per product phase.
  for (int b = 0; b < (int)p.buckets.size(); ++b) {
    const BucketPlan& bp = p.buckets[b];
    if (!bp.small) continue;
    p.small.push_back(b);
    const int64_t ti = bp.mp / kSmallTile, tj = bp.np / kSmallTile, cnt = (int64_t)bp.slices.size();
    p.small_wgs[0] += cnt * ti * ti;
    p.small_wgs[1] += cnt * ti * ti;
    p.small_wgs[2] += cnt * ti * tj;
  }
  if (!p.small.empty()) {
    if (p.small_wgs[2] >= (int64_t(1) << 31)) {
      *err = "too many small product tiles in one plan";
      return MUON_ERR_UNSUPPORTED;
    }
    p.launches_per_ns += 3;
    p.off_small_params = ws.take(p.small.size() * sizeof(SmallBucket));
  }
  // The other streamed buckets share one launch per product phase too.  The
  // output tile of a phase is 128, or 64 when the whole group has fewer
  // 128-tiles than the chip has CUs; each output entry takes its k steps in
  // the same order for either size, so the choice changes no bit.
  int64_t t128[3] = {0, 0, 0};
  for (int b = 0; b < (int)p.buckets.size(); ++b) {
    const BucketPlan& bp = p.buckets[b];
    if (bp.path != MUON_PATH_STREAM || bp.big || bp.small) continue;
    p.mid.push_back(b);
    const int64_t ti = bp.mp / 128, tj = bp.np / 128, cnt = (int64_t)bp.slices.size();
    t128[0] += cnt * ti * ti;
    t128[1] += cnt * ti * ti;
    t128[2] += cnt * ti * tj;
  }
  if (!p.mid.empty()) {
    // Longest contractions first, so the launch does not end on them: the
    // Gram phase contracts over n (the other phases over m).
    std::stable_sort(p.mid.begin(), p.mid.end(), [&](int a, int b) { return p.buckets[a].np > p.buckets[b].np; });
    for (int ph = 0; ph < 3; ++ph) {
      p.mid_bt[ph] = t128[ph] < kMidMinTiles ? 64 : 128;
      p.mid_wgs[ph] = p.mid_bt[ph] == 64 ? 4 * t128[ph] : t128[ph];
      if (p.mid_wgs[ph] >= (int64_t(1) << 31)) {
        *err = "too many product tiles in one plan";
        return MUON_ERR_UNSUPPORTED;
      }
    }
    p.launches_per_ns += 3;
    p.off_mid_params = ws.take(p.mid.size() * sizeof(SmallBucket));
  }
  // Large buckets share one launch per product phase.
  for (int b = 0; b < (int)p.buckets.size(); ++b)
    if (p.buckets[b].big) p.big.push_back(b);
  if (p.big.size() > 255) {
    *err = "too many distinct large shapes in one plan (at most 255)";
    return MUON_ERR_UNSUPPORTED;
  }
  if (!p.big.empty()) {
    p.launches_per_ns += 3;
    p.off_big_params = ws.take(p.big.size() * sizeof(BigBucket));
    for (int ph = 0; ph < 3; ++ph) {
      p.big_tab[ph] = big_table(p, ph);
      p.off_big_tab[ph] = ws.take(p.big_tab[ph].size() * sizeof(BigTile));
    }
  }
  p.ws_total = align_up(ws.top, 256);
  if (p.workspace_limit != 0 && p.ws_total > p.workspace_limit) {
    std::snprintf(buf, sizeof buf, "workspace needs %llu bytes, limit is %llu",
                  (unsigned long long)p.ws_total, (unsigned long long)p.workspace_limit);
    *err = buf;
    return MUON_ERR_OOM;
  }
  *out = std::move(p);
  return MUON_OK;
}

std::vector<BigTile> big_table(const Plan& p, int phase) {
  constexpr int kXcd = 8;
  struct Block {
    int64_t k;     // contraction length of every tile in the block
    int64_t work;  // k per full tile, k / 2 per half tile (measured: about 0.6 k)
    std::vector<BigTile> tiles;
  };
  std::vector<Block> blocks;
  for (int bi = 0; bi < (int)p.big.size(); ++bi) {
    const BucketPlan& bp = p.buckets[p.big[bi]];
    const int tm = (int)(bp.mp / kBigTile);
    const int tn = phase == 2 ? (int)(bp.np / kBigTile) : tm;
    const bool sym = phase != 2;
    const int64_t k = big_k_over_m(phase == 0 ? bp.n : bp.m);
    // Blocks of 32 tiles, 4 rows x 8 columns.  A slice of at most 8 row tiles
    // is cut whole along its rows instead, where a 4-row block would leave a
    // ragged remainder: an apply takes all its row tiles x 4 columns, a
    // symmetric product its whole upper triangle as one block (measured on
    // the 6 x 8 and 6 x 6 grids of [1408,2048]: 5% and 2% faster phases).
    // A larger symmetric product takes the 8 x 8 triangles on the diagonal
    // (36 tiles that share 8 panels) and cuts the squares above them into
    // 4 x 8 blocks (the Gram measured 0.7% faster than with 4 x 8 blocks
    // throughout).
    const int kRows = tm <= 8 ? 8 : 4, kCols = sym && tm <= 8 ? 8 : 32 / kRows;
    // The kernel's half tiles (symmetric products only): the output tile row
    // is the last one and holds at most 128 rows inside m (on such a slice
    // the kernel takes the table's column index as the row).
    const bool half_row = sym && bp.m - (int64_t)(tm - 1) * kBigTile <= 128;
    auto add_block = [&](int z, int i0, int i1, int j0, int j1) {
      Block blk{k, 0, {}};
      for (int i = i0; i < i1 && i < tm; ++i)
        for (int j = j0; j < j1 && j < tn; ++j)
          if (!sym || j >= i) {
            blk.tiles.push_back(BigTile{(uint32_t)bi << 24 | (uint32_t)z, (uint32_t)i | (uint32_t)j << 16});
            blk.work += half_row && j == tm - 1 ? k / 2 : k;
          }
      if (!blk.tiles.empty()) blocks.push_back(std::move(blk));
    };
    for (int z = 0; z < (int)bp.slices.size(); ++z) {
      if (sym && tm > 8) {
        for (int d0 = 0; d0 < tm; d0 += 8) add_block(z, d0, d0 + 8, d0, d0 + 8);
        for (int i0 = 0; i0 < tm; i0 += 8)
          for (int j0 = i0 + 8; j0 < tn; j0 += 8) {
            add_block(z, i0, i0 + 4, j0, j0 + 8);
            add_block(z, i0 + 4, i0 + 8, j0, j0 + 8);
          }
        continue;
      }
      for (int i0 = 0; i0 < tm; i0 += kRows)
        for (int j0 = sym ? (i0 / kCols) * kCols : 0; j0 < tn; j0 += kCols)
          add_block(z, i0, i0 + kRows, j0, j0 + kCols);
    }
  }
  std::stable_sort(blocks.begin(), blocks.end(), [](const Block& x, const Block& y) { return x.k > y.k; });
  std::vector<BigTile> part[kXcd];
  int64_t load[kXcd] = {};
  for (const Block& blk : blocks) {
    int x = 0;
    for (int i = 1; i < kXcd; ++i)
      if (load[i] < load[x]) x = i;
    part[x].insert(part[x].end(), blk.tiles.begin(), blk.tiles.end());
    load[x] += blk.work;
  }
  size_t len = 0;
  for (auto& v : part) len = std::max(len, v.size());
  std::vector<BigTile> t;
  t.reserve(len * kXcd);
  for (auto& v : part) {
    v.resize(len, BigTile{kNoTile, 0});
    t.insert(t.end(), v.begin(), v.end());
  }
  return t;
}

void fill_info(const Plan& p, muon_plan_info_t* info) {
  std::memset(info, 0, sizeof(*info));
  info->n_params = p.n_params;
  info->n_matrices = (int)p.slices.size();
  info->n_buckets = (int)p.buckets.size();
  info->mode = p.mode;
  info->workspace_bytes = p.ws_total;
  info->launches_fixed = p.launches_fixed;
  info->launches_per_ns = p.launches_per_ns;
  for (int i = 0; i < (int)p.buckets.size() && i < MUON_MAX_BUCKETS; ++i) {
    const BucketPlan& b = p.buckets[i];
    muon_bucket_info_t& o = info->buckets[i];
    o.m = b.m;
    o.n = b.n;
    o.count = (int)b.slices.size();
    o.n_transposed = b.n_transposed;
    o.path = b.path;
    o.chunks = b.n_chunks;
    o.workspace_bytes = b.ws_bytes;
  }
}

}  // namespace muon
