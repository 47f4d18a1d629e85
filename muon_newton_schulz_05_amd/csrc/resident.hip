// resident.hip -- the whole Muon step for skinny slices (m <= 32) in one launch.
//
// The pages measure that small matrices leave the matrix unit idle while host
// dispatch, small allocations and stream syncs dominate ("MindSpore
// HyperParallel X 盘古,Muon优化器实现6倍性能跃升", sections 三大性能挑战 and
// 矩阵融合优化, with 74 parameters of [24, 10240] as the example).  Here a
// slice never leaves the chip between rounds: a cluster of workgroups splits
// its n columns, keeps its part of X in registers for all k rounds and only
// exchanges the 32 x 32 partial Gram matrices (the split-over-columns form of
// "关于分布式Muon的想法整合及讨论" §6, where parts add up their sums of squares and
// their Gram contributions).
//
// Register layout of a 32-column tile of X ("column layout"): lane l holds
// column (l % 32) and the 16 rows rho(r, l) = 8 (r / 4) + 4 (l / 32) + r % 4,
// r = 0..15, which is the row set of the 32x32 matrix-core output layout.  So
//   X' = P X     keeps the column layout (X is the B operand, P the A operand
//                loaded with the same row permutation), and
//   X^T E        (E a 0/1 selection matrix) turns it into the row layout
//                (lane l holds row l % 32), exactly, which is what the Gram
//                product X X^T needs as both of its operands.
//
// Synchronisation: the launch is cooperative, so every workgroup of a cluster
// is resident; arrivals are counted per slice with agent-scope release /
// acquire atomics.  Every wait is bounded: after spin_limit polls the
// workgroup records an error bit and carries on, so the grid always drains.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

constexpr int kThreads = kResidentWaves * 64;

struct ResArgs {
  const DevMat* mats;
  const PtrEntry* ptrs;
  const DevScalars* sc;
  float* gram_parts;       // two slot sets of slot_stride floats each
  int64_t slot_stride;     // count * cluster * 1024
  double* sq_parts;
  uint32_t* ctrs;
  uint32_t* err;
  int m, n;
  int cluster, tiles_per_wg;
  int mat_base, grid_real, grid_pad;
  int ns_steps;
  uint32_t spin_limit;
};

__device__ __forceinline__ int rho(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Arrive at exchange `round` of a slice and wait for the whole cluster.
__device__ __forceinline__ void cluster_sync(uint32_t* ctr, uint32_t target, uint32_t* err,
                                             uint32_t spin_limit) {
  __threadfence();  // publish this thread's partial results at agent scope
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > spin_limit) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

template <int TPW, bool BF16>
__global__ __launch_bounds__(kThreads) void k_resident(ResArgs a) {
  __shared__ float red[kResidentWaves][1024];
  __shared__ float As[32][33];
  __shared__ float Bs[32][33];
  __shared__ double sq_red[kResidentWaves];
  __shared__ float sh_scale;

  const int per_xcd = a.grid_pad / 8;
  const int linear = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;  // keep a cluster on one XCD
  if (linear >= a.grid_real) return;
  const int local = linear / a.cluster, member = linear % a.cluster;
  const int zi = a.mat_base + local;
  const DevMat d = a.mats[zi];
  const PtrEntry pe = a.ptrs[d.param];
  const float beta = a.sc->beta, ca = a.sc->a, cb = a.sc->b, cc = a.sc->c, lr = a.sc->lr;
  const float eps = a.sc->eps;
  const int m = a.m, n = a.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int ntiles = (n + 31) / 32;
  const int t_begin = member * a.tiles_per_wg;
  const int t_end = min(t_begin + a.tiles_per_wg, ntiles);
  const int ns = a.ns_steps;
  const bool tr_store = d.transposed != 0;

  // Slice bases (uniform) and 32-bit element offsets: element (i, j) of the
  // oriented slice sits at lane_base(j) + row_off(r) for i = rho(r, h).
  // Loads use a uniform base plus a 32-bit byte offset.
  const MUON_GLOBAL char* const Mb = as_global(reinterpret_cast<const char*>(pe.m + d.slice_off));
  const int gdt = d.gdtype, pdt = d.pdtype;
  const MUON_GLOBAL char* const Gb = as_global(static_cast<const char*>(pe.g) + d.slice_off * (gdt ? 2 : 4));
  const MUON_GLOBAL char* const Wb = as_global(static_cast<const char*>(pe.w) + d.slice_off * (pdt ? 2 : 4));
  auto row_off = [&](int r) -> uint32_t {
    const uint32_t i = 8 * (r >> 2) + (r & 3);
    return tr_store ? i : i * (uint32_t)n;
  };
  // The per-tile base is passed through an empty asm so that the compiler
  // recomputes addresses where they are used instead of keeping every
  // address of every tile live across the whole iteration.
  auto lane_base = [&](int j) -> uint32_t {
    uint32_t b = tr_store ? (uint32_t)j * (uint32_t)m + 4u * h : 4u * h * (uint32_t)n + (uint32_t)j;
    asm volatile("" : "+v"(b));
    return b;
  };
  auto ldm = [&](uint32_t o) -> float { return *reinterpret_cast<const MUON_GLOBAL float*>(Mb + (o << 2)); };
  auto stm = [&](uint32_t o, float v) {
    *reinterpret_cast<MUON_GLOBAL float*>(const_cast<MUON_GLOBAL char*>(Mb) + (o << 2)) = v;
  };
  // Typed loads/stores; callers pick the storage type once per phase.
  auto ld16or32 = [](const MUON_GLOBAL char* base, uint32_t o, auto is16) -> float {
    if constexpr (decltype(is16)::value) return from_bf16(*reinterpret_cast<const MUON_GLOBAL uint16_t*>(base + (o << 1)));
    else return *reinterpret_cast<const MUON_GLOBAL float*>(base + (o << 2));
  };
  auto st16or32 = [](const MUON_GLOBAL char* base, uint32_t o, float v, auto is16) {
    MUON_GLOBAL char* w = const_cast<MUON_GLOBAL char*>(base);
    if constexpr (decltype(is16)::value) *reinterpret_cast<MUON_GLOBAL uint16_t*>(w + (o << 1)) = to_bf16(v);
    else *reinterpret_cast<MUON_GLOBAL float*>(w + (o << 2)) = v;
  };
  using F32 = std::integral_constant<bool, false>;
  using B16 = std::integral_constant<bool, true>;

  // X tiles in registers (column layout): bf16 pairs (r, r + 1) packed, four
  // registers per contraction block g (rows r = 8g .. 8g+7) in xv[q][g]; or
  // float32 xf[q][r].
  u32x4_t xv[BF16 ? TPW : 1][2];
  float xf[BF16 ? 1 : TPW][16];
  auto xop = [&](int q, int g) { return __builtin_bit_cast(bf16x8_t, xv[q][g]); };
  auto xval = [&](int q, int r) -> float {
    const uint32_t w = xv[q][r >> 3][(r >> 1) & 3];
    return (r & 1) ? bf16_hi(w) : bf16_lo(w);
  };
  auto xset = [&](int q, const float* v) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      xv[q][g] = u32x4_t{pack_bf16x2(v[8 * g], v[8 * g + 1]), pack_bf16x2(v[8 * g + 2], v[8 * g + 3]),
                         pack_bf16x2(v[8 * g + 4], v[8 * g + 5]), pack_bf16x2(v[8 * g + 6], v[8 * g + 7])};
  };

  // 0/1 selection operand of the transposing product X^T E.
  bf16x8_t esel[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int t = 0; t < 8; ++t) esel[g][t] = (__bf16)(rho(8 * g + t, h) == col ? 1.f : 0.f);

  // ---- momentum, sum of squares, unscaled X0 = M_new ------------------------------
  // All loads of a tile are issued before any use; lanes outside the slice
  // read element 0 (always valid) and discard it.
  float sq = 0.f;
  auto phase0 = [&](auto gtype) {
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int tile = t_begin + wave + kResidentWaves * q;
      const int j = tile * 32 + col;
      const bool colok = tile < t_end && j < n;
      const uint32_t lb = lane_base(j);
      float v[16];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t off[8];
        float mo[8], gv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 8 * half + u;
          const bool ok = colok && rho(r, h) < m;
          off[u] = ok ? lb + row_off(r) : 0u;
          mo[u] = ldm(off[u]);
          gv[u] = ld16or32(Gb, off[u], gtype);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 8 * half + u;
          const bool ok = colok && rho(r, h) < m;
          const float mn = ok ? fmaf(beta, mo[u], gv[u]) : 0.f;
          if (ok) stm(off[u], mn);
          sq = fmaf(mn, mn, sq);
          v[r] = mn;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (BF16) {
        xset(q, v);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) xf[q][r] = v[r];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (gdt) phase0(B16{});
  else phase0(F32{});

  // Gram partial of one tile, accumulated per wave.
  auto gram_tile = [&](int q, f32x16_t& acc) {
    f32x16_t tr = {};
    if constexpr (BF16) {
      tr = mfma_bf16(xop(q, 0), esel[0], tr);  // X^T E: exact transpose into the row layout
      if (m > 16) tr = mfma_bf16(xop(q, 1), esel[1], tr);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const bf16x8_t rt = as_bf16x8(pack_bf16x2(tr[8 * g], tr[8 * g + 1]), pack_bf16x2(tr[8 * g + 2], tr[8 * g + 3]),
                                      pack_bf16x2(tr[8 * g + 4], tr[8 * g + 5]), pack_bf16x2(tr[8 * g + 6], tr[8 * g + 7]));
        acc = mfma_bf16(rt, rt, acc);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (rho(r, 0) >= m) continue;
        tr = mfma_f32(xf[q][r], rho(r, h) == col ? 1.f : 0.f, tr);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc = mfma_f32(tr[r], tr[r], acc);
    }
  };

  // Reduce the waves' Gram partials and sums of squares, publish the
  // workgroup's partials, wait for the cluster, then build A and
  // B = b A + c A^2 in LDS (float32, fixed order).
  auto exchange = [&](int round, const f32x16_t& acc, bool with_gram, bool with_sq) {
    if (with_gram) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][rho(r, h) * 32 + col] = acc[r];
    }
    if (with_sq) {
      const float ws = wave_sum(sq);
      if (lane == 0) sq_red[wave] = (double)ws;
    }
    __syncthreads();
    // Two slot sets by round parity: a member that has read round r and moved
    // on writes round r + 1 elsewhere while slower members still read round r;
    // it cannot reach round r + 2 before they have arrived at r + 1.
    float* const slots = a.gram_parts + (int64_t)(round & 1) * a.slot_stride;
    float* my_part = slots + ((int64_t)zi * a.cluster + member) * 1024;
    if (with_gram) {
      for (int e = tid; e < 1024; e += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kResidentWaves; ++w) s += red[w][e];
        my_part[e] = s;
      }
    }
    if (with_sq && tid == 0) {
      double s = 0.0;
      for (int w = 0; w < kResidentWaves; ++w) s += sq_red[w];
      a.sq_parts[(int64_t)zi * a.cluster + member] = s;
    }
    cluster_sync(a.ctrs + zi, (uint32_t)(a.cluster * (round + 1)), a.err, a.spin_limit);
    if (with_sq && tid == 0) {
      double s = 0.0;
      for (int p = 0; p < a.cluster; ++p) s += a.sq_parts[(int64_t)zi * a.cluster + p];
      sh_scale = (float)(1.0 / (sqrt(s) + (double)eps));
    }
    __syncthreads();
    if (with_gram) {
      const float s2 = with_sq ? sh_scale * sh_scale : 1.f;
      const float* parts = slots + (int64_t)zi * a.cluster * 1024;
      for (int e = tid; e < 1024; e += kThreads) {
        float s = 0.f;
        for (int p = 0; p < a.cluster; ++p) s += parts[(int64_t)p * 1024 + e];
        As[e >> 5][e & 31] = s * s2;
      }
      __syncthreads();
      for (int e = tid; e < 1024; e += kThreads) {
        const int i = e >> 5, j = e & 31;
        float s = 0.f;
#pragma unroll 8
        for (int k = 0; k < 32; ++k) s = fmaf(As[i][k], As[k][j], s);
        Bs[i][j] = cb * As[i][j] + cc * s;
      }
      __syncthreads();
    }
  };

  {
    f32x16_t acc = {};
    if (ns > 0) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        if (t_begin + wave + kResidentWaves * q < t_end) gram_tile(q, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    exchange(0, acc, ns > 0, true);
  }
  const float s0 = sh_scale;

  // W <- W - lr * O for one tile, O given in the column layout.
  auto update_tile = [&](int q, const float* o, auto wtype) {
    const int tile = t_begin + wave + kResidentWaves * q;
    const int j = tile * 32 + col;
    const bool colok = tile < t_end && j < n;
    const uint32_t lb = lane_base(j);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t off[8];
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 8 * half + u;
        const bool ok = colok && rho(r, h) < m;
        off[u] = ok ? lb + row_off(r) : 0u;
        w[u] = ld16or32(Wb, off[u], wtype);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 8 * half + u;
        const bool ok = colok && rho(r, h) < m;
        if (ok) st16or32(Wb, off[u], w[u] - lr * o[8 * half + u], wtype);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (ns == 0) {
    // O = s M_new, read back at full precision.
    auto run = [&](auto wtype) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int tile = t_begin + wave + kResidentWaves * q;
        const int j = tile * 32 + col;
        const bool colok = tile < t_end && j < n;
        const uint32_t lb = lane_base(j);
        float o[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = colok && rho(r, h) < m;
          o[r] = s0 * ldm(ok ? lb + row_off(r) : 0u);
        }
        update_tile(q, o, wtype);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (pdt) run(B16{});
    else run(F32{});
    return;
  }

  // P operand registers: row permutation rho on the contraction index.
  bf16x8_t phi[2], plo[2];
  float pf[BF16 ? 1 : 16];
  auto load_p = [&]() {
    if constexpr (BF16) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float v = Bs[col][rho(8 * g + t, h)];
          const __bf16 hi = (__bf16)v;
          phi[g][t] = hi;
          plo[g][t] = (__bf16)(v - (float)hi);
        }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) pf[r] = Bs[col][rho(r, h)];
    }
  };
  // dx = scale * (a X + P X) for tile q.
  auto px_tile = [&](int q, float scale, float* dxo) {
    f32x16_t dx = {};
    if constexpr (BF16) {
      dx = mfma_bf16(phi[0], xop(q, 0), dx);
      dx = mfma_bf16(plo[0], xop(q, 0), dx);
      if (m > 16) {
        dx = mfma_bf16(phi[1], xop(q, 1), dx);
        dx = mfma_bf16(plo[1], xop(q, 1), dx);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (rho(r, 0) >= m) continue;
        dx = mfma_f32(pf[r], xf[q][r], dx);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float xold;
      if constexpr (BF16) xold = xval(q, r);
      else xold = xf[q][r];
      dxo[r] = scale * fmaf(ca, xold, dx[r]);
    }
  };

  // Rounds 0 .. ns-2: X <- a X + P X in registers, Gram partial of the new X.
  for (int it = 0; it + 1 < ns; ++it) {
    const float scale = it == 0 ? s0 : 1.f;
    load_p();
    f32x16_t acc = {};
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      if (t_begin + wave + kResidentWaves * q < t_end) {
        float v[16];
        px_tile(q, scale, v);
        if constexpr (BF16) {
          xset(q, v);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) xf[q][r] = v[r];
        }
        gram_tile(q, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    exchange(it + 1, acc, true, false);
  }

  // Last round: W <- W - lr (a X + P X), straight from the registers.
  {
    const float scale = ns == 1 ? s0 : 1.f;
    load_p();
    auto run = [&](auto wtype) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        if (t_begin + wave + kResidentWaves * q < t_end) {
          float v[16];
          px_tile(q, scale, v);
          update_tile(q, v, wtype);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (pdt) run(B16{});
    else run(F32{});
  }
}

template <int TPW, bool BF16>
hipError_t launch_variant(const ResidentLaunch& L, hipStream_t s) {
  ResArgs a;
  a.mats = L.mats;
  a.ptrs = L.ptrs;
  a.sc = L.sc;
  a.gram_parts = L.gram_parts;
  a.slot_stride = (int64_t)L.count * L.cluster * 1024;
  a.sq_parts = L.sq_parts;
  a.ctrs = L.ctrs;
  a.err = L.err;
  a.m = L.m;
  a.n = L.n;
  a.cluster = L.cluster;
  a.tiles_per_wg = L.tiles_per_wg;
  a.mat_base = L.mat_base;
  a.grid_real = L.n_mats * L.cluster;
  a.grid_pad = (a.grid_real + 7) / 8 * 8;
  a.ns_steps = L.ns_steps;
  a.spin_limit = L.spin_limit;
  void* args[] = {&a};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_resident<TPW, BF16>),
                                    dim3(a.grid_pad), dim3(kThreads), args, 0, s);
}

template <int TPW, bool BF16>
int occupancy_variant() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, &k_resident<TPW, BF16>, kThreads, 0) !=
      hipSuccess)
    return 0;
  return blocks;
}

}  // namespace

hipError_t launch_resident(const ResidentLaunch& L, hipStream_t s) {
  if (L.bf16) {
    switch (L.tpw) {
      case 1: return launch_variant<1, true>(L, s);
      case 2: return launch_variant<2, true>(L, s);
      case 4: return launch_variant<4, true>(L, s);
      case 8: return launch_variant<8, true>(L, s);
      case 14: return launch_variant<14, true>(L, s);
    }
  } else {
    switch (L.tpw) {
      case 1: return launch_variant<1, false>(L, s);
      case 2: return launch_variant<2, false>(L, s);
      case 4: return launch_variant<4, false>(L, s);
      case 8: return launch_variant<8, false>(L, s);
    }
  }
  return hipErrorInvalidValue;
}

int resident_occupancy(int tpw, int bf16) {
  if (bf16) {
    switch (tpw) {
      case 1: return occupancy_variant<1, true>();
      case 2: return occupancy_variant<2, true>();
      case 4: return occupancy_variant<4, true>();
      case 8: return occupancy_variant<8, true>();
      case 14: return occupancy_variant<14, true>();
    }
  } else {
    switch (tpw) {
      case 1: return occupancy_variant<1, false>();
      case 2: return occupancy_variant<2, false>();
      case 4: return occupancy_variant<4, false>();
      case 8: return occupancy_variant<8, false>();
    }
  }
  return 0;
}

}  // namespace muon
