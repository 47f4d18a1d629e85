// skinny.hip -- the Muon step for slices with m <= 32 rows (after orientation).
//
// The pages single out exactly this regime: many small matrices such as
// [24, 10240], where the matrix unit is nearly idle and host dispatch and
// memory traffic dominate ("MindSpore HyperParallel X 盘古,Muon优化器实现6倍性能跃升",
// sections 三大性能挑战 and 矩阵融合优化, Fig. 6-7).
//
// Newton-Schulz here runs in the space of the m x m Gram matrix.  With
// X_{t+1} = P_t X_t and P_t = a I + b A_t + c A_t^2 a polynomial in
// A_t = X_t X_t^T, P_t commutes with A_t, so
//     A_{t+1} = P_t A_t P_t = P_t^2 A_t   and   X_k = (P_{k-1} ... P_0) X_0.
// Only the first Gram matrix needs the n columns; every later round is
// m x m arithmetic, and X_k is one product Q X_0 at the end.  The result is
// the iteration of "关于分布式Muon的想法整合及讨论" §2 and §6 (Gram matrix
// recomputed every round, normalisation by the whole-matrix sum of squares);
// only the order of the floating-point operations differs.
//
// Three kernels per bucket, all batched over the bucket's slices:
//   k_skinny_gram   momentum M <- beta M + G (stored), and per 256-column
//                   chunk the sum of squares and the Gram partial of X0 = M,
//                   on the matrix cores (split-K over the long dimension);
//   k_skinny_poly   (skinny_poly.hip) per slice: s = 1/(||M||_F + eps),
//                   A0 = s^2 sum of the partials, the k-round recurrence in
//                   float64, Qs = s Q;
//   k_skinny_apply  O = Qs M (matrix cores), W <- W - lr O.
// Chunks are fixed by n alone, so a slice's arithmetic does not depend on the
// batch it is fused into.  Both memory passes stream 16-byte accesses in
// storage order and turn them around in LDS, so one code path serves slices
// stored as [m, n] and as [n, m].
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCols = kSkinnyChunk;            // columns per chunk
constexpr int kStride = kCols + 4;             // LDS row stride in floats
constexpr int kChunks = 32 * kCols / 4 / kThreads;  // 4-element pieces per thread (m = 32)
constexpr int kTilesPerWave = kCols / 32 / kWaves;

using F32 = std::integral_constant<bool, false>;
using B16 = std::integral_constant<bool, true>;

__device__ __forceinline__ int rho(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <typename Is16>
__device__ __forceinline__ float ld_elem(const char* base, int64_t o) {
  if constexpr (Is16::value) return from_bf16(*reinterpret_cast<const MUON_GLOBAL uint16_t*>(as_global(base) + 2 * o));
  else return *reinterpret_cast<const MUON_GLOBAL float*>(as_global(base) + 4 * o);
}
template <typename Is16>
__device__ __forceinline__ void st_elem(char* base, int64_t o, float v) {
  if constexpr (Is16::value) *reinterpret_cast<MUON_GLOBAL uint16_t*>(as_global(base) + 2 * o) = to_bf16(v);
  else *reinterpret_cast<MUON_GLOBAL float*>(as_global(base) + 4 * o) = v;
}
template <typename Is16>
__device__ __forceinline__ void ld_vec4(const char* base, int64_t o, float* v) {
  if constexpr (Is16::value) {
    const u32x2_t w = *reinterpret_cast<const MUON_GLOBAL u32x2_t*>(as_global(base) + 2 * o);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  } else {
    const f32x4_t w = *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(base) + 4 * o);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
}
template <typename Is16>
__device__ __forceinline__ void st_vec4(char* base, int64_t o, const float* v) {
  if constexpr (Is16::value) {
    *reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(base) + 2 * o) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(base) + 4 * o) = f32x4_t{v[0], v[1], v[2], v[3]};
  }
}

// The storage of one chunk (oriented columns [c0, c0 + cw) of an m-row
// slice), cut into 4-element pieces dealt to the threads.
struct ChunkMap {
  int m, n, c0, cw;
  bool tr;        // slice stored as [n, m]
  bool vec_ok;    // 16-byte accesses are aligned
  uint32_t magic; // ceil(2^32 / m) for m >= 2: exact division of offsets < 2^14
  int per_row;    // [m, n] storage: pieces per row of the chunk
  int total;      // pieces in the chunk

  __device__ void init(int m_, int n_, int c0_, int cw_, bool tr_, int64_t slice_off) {
    m = m_; n = n_; c0 = c0_; cw = cw_; tr = tr_;
    vec_ok = (slice_off & 3) == 0 && (tr || (n & 3) == 0);
    magic = m >= 2 ? (uint32_t)((((uint64_t)1 << 32) + (uint64_t)m - 1) / (uint64_t)m) : 0u;
    per_row = (cw + 3) >> 2;
    total = tr ? (cw * m + 3) >> 2 : m * per_row;
  }
  __device__ int divm(int e) const { return m == 1 ? e : (int)__umulhi((uint32_t)e, magic); }
  // Piece v: storage offset of its first element, valid count, and the
  // oriented (row, column-in-chunk) of the first element.
  __device__ void piece(int v, int64_t& off, int& cnt, int& i0, int& j0) const {
    if (!tr) {
      const int i = per_row == kCols / 4 ? v / (kCols / 4) : v / per_row;
      const int jj = (v - i * per_row) * 4;
      off = (int64_t)i * n + c0 + jj;
      cnt = min(4, cw - jj);
      i0 = i;
      j0 = jj;
    } else {
      const int e0 = 4 * v;
      const int jj = divm(e0);
      off = (int64_t)c0 * m + e0;
      cnt = min(4, cw * m - e0);
      i0 = e0 - jj * m;
      j0 = jj;
    }
  }
  // Oriented position of element u of a piece that starts at (i0, j0).
  __device__ void pos(int i0, int j0, int u, int& i, int& j) const {
    if (!tr) {
      i = i0;
      j = j0 + u;
    } else {
      const int e = i0 + u;
      const int q = divm(e);
      i = e - q * m;
      j = j0 + q;
    }
  }
};

// Zero the part of a staging block that a chunk does not fill: rows >= m,
// and columns >= cw of the other rows.
__device__ __forceinline__ void zero_unfilled(float (*st)[kStride], int m, int cw, int tid) {
  for (int e = tid; e < (32 - m) * kCols; e += kThreads) st[m + e / kCols][e % kCols] = 0.f;
  if (cw < kCols) {
    const int w = kCols - cw;
    for (int e = tid; e < m * w; e += kThreads) st[e / w][cw + e % w] = 0.f;
  }
}

// ------------------------------------------------------------------ gram
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_skinny_gram(SkinnyLaunch a) {
  __shared__ __attribute__((aligned(16))) float st[32][kStride];
  __shared__ float wsq[kWaves];
  // The waves' Gram partials (float64) reuse the staging block once it has been read.
  double (*red)[1024] = reinterpret_cast<double (*)[1024]>(&st[0][0]);
  static_assert(kWaves * 1024 * 2 <= 32 * kStride, "reduction buffer must fit the staging block");

  const int z = blockIdx.y, chunk = blockIdx.x;
  const DevMat d = a.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float beta = a.sc_out ? a.sv.beta : a.sc->beta;
  const bool nesterov = (a.sc_out ? a.sv.nesterov : a.sc->nesterov) != 0;
  if (a.sc_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.sc_out = a.sv;
  const int m = a.m, n = a.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  ChunkMap cm;
  cm.init(m, n, chunk * kCols, min(kCols, n - chunk * kCols), d.transposed != 0, d.slice_off);
  char* const Mb = reinterpret_cast<char*>(pe.m + d.slice_off);
  const char* const Gb = static_cast<const char*>(pe.g) + d.slice_off * (d.gdtype ? 2 : 4);

  zero_unfilled(st, m, cm.cw, tid);

  // Issue every load of the chunk, then M <- beta M + G, store M, stage the
  // matrix that is orthogonalised: M, or G + beta M with Nesterov momentum.
  auto pass = [&](auto gtype) {
    using GT = decltype(gtype);
    float lm[kChunks][4], lg[kChunks][4];
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      int64_t off = 0;
      int cnt = 0, i0 = 0, j0 = 0;
      if (v < cm.total) cm.piece(v, off, cnt, i0, j0);
      if (cnt == 4 && cm.vec_ok) {
        ld_vec4<F32>(Mb, off, lm[k]);
        ld_vec4<GT>(Gb, off, lg[k]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lm[k][u] = u < cnt ? ld_elem<F32>(Mb, off + u) : 0.f;
          lg[k][u] = u < cnt ? ld_elem<GT>(Gb, off + u) : 0.f;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      if (v >= cm.total) continue;
      int64_t off;
      int cnt, i0, j0;
      cm.piece(v, off, cnt, i0, j0);
      float mn[4], xs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mn[u] = fmaf(beta, lm[k][u], lg[k][u]);
        xs[u] = nesterov ? fmaf(beta, mn[u], lg[k][u]) : mn[u];
      }
      if (cnt == 4 && cm.vec_ok) {
        st_vec4<F32>(Mb, off, mn);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (u < cnt) st_elem<F32>(Mb, off + u, mn[u]);
      }
      if (!cm.tr && cnt == 4) {
        *reinterpret_cast<f32x4_t*>(&st[i0][j0]) = f32x4_t{xs[0], xs[1], xs[2], xs[3]};
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u >= cnt) break;
          int i, j;
          cm.pos(i0, j0, u, i, j);
          st[i][j] = xs[u];
        }
      }
    }
  };
  if (d.gdtype) pass(B16{});
  else pass(F32{});
  __syncthreads();

  // Sum of squares in oriented order: thread t owns columns t, t + 256.
  float sq = 0.f;
  for (int j = tid; j < kCols; j += kThreads)
    for (int i = 0; i < m; ++i) sq = fmaf(st[i][j], st[i][j], sq);
  sq = wave_sum(sq);
  if (lane == 0) wsq[wave] = sq;

  // Gram partial: lane l holds row l % 32; both operands are the same rows.
  // Each 32-column tile is accumulated in float32 on the matrix cores and
  // added into a float64 running sum, so the partial's rounding does not
  // grow with the chunk width.
  double accd[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) accd[r] = 0.0;
  const int row = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int q = 0; q < kTilesPerWave; ++q) {
    const int t = wave + kWaves * q;
    if (t * 32 >= cm.cw) break;
    f32x16_t acc = {};
    if constexpr (BF16) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int c = t * 32 + g * 16 + kh * 8;
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&st[row][c]);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(&st[row][c + 4]);
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          hw[u] = pack_bf16x2(x[2 * u], x[2 * u + 1]);
          lw[u] = pack_bf16x2(x[2 * u] - bf16_lo(hw[u]), x[2 * u + 1] - bf16_hi(hw[u]));
        }
        const bf16x8_t xh = as_bf16x8(hw[0], hw[1], hw[2], hw[3]);
        const bf16x8_t xl = as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
        acc = mfma_bf16(xh, xh, acc);
        acc = mfma_bf16(xh, xl, acc);
        acc = mfma_bf16(xl, xh, acc);
        acc = mfma_bf16(xl, xl, acc);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const float x = st[row][t * 32 + 2 * s + kh];
        acc = mfma_f32(x, x, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) accd[r] += (double)acc[r];
  }
  // Output layout: lane l, register r -> row rho(r, l / 32), column l % 32.
  __syncthreads();  // every wave is done reading the staging block
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][rho(r, kh) * 32 + row] = accd[r];
  __syncthreads();
  const int64_t part = (int64_t)z * a.n_chunks + chunk;
  for (int e = tid; e < m * m; e += kThreads) {  // the m x m block, row-major
    const int i = e / m, j = e - i * m;
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w][i * 32 + j];
    a.gram_parts[part * m * m + e] = s;
  }
  if (tid == 0) a.sq_parts[part] = ((wsq[0] + wsq[1]) + wsq[2]) + wsq[3];
}

// ------------------------------------------------------------------ apply
// NEST: Nesterov momentum (X = G + beta M); chosen at launch from the plan so
// that the plain kernel carries no second code path.
template <bool BF16, bool NEST>
__global__ __launch_bounds__(kThreads) void k_skinny_apply(SkinnyLaunch a) {
  __shared__ __attribute__((aligned(16))) float st[32][kStride];
  __shared__ float qs[32][33];

  const int z = blockIdx.y, chunk = blockIdx.x;
  const DevMat d = a.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float lr = a.sc->lr, decay = a.sc->decay, beta = a.sc->beta;
  const int m = a.m, n = a.n;
  const float lrf = lr * update_factor(a.sc->scale_mode, m, n, d.transposed);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  ChunkMap cm;
  cm.init(m, n, chunk * kCols, min(kCols, n - chunk * kCols), d.transposed != 0, d.slice_off);
  const char* const Mb = reinterpret_cast<const char*>(pe.m + d.slice_off);
  const char* const Gb = static_cast<const char*>(pe.g) + d.slice_off * (d.gdtype ? 2 : 4);
  char* const Wb = static_cast<char*>(pe.w) + d.slice_off * (d.pdtype ? 2 : 4);

  for (int e = tid; e < 1024; e += kThreads) qs[e >> 5][e & 31] = a.qs[(int64_t)z * 1024 + e];

  // gmode: 0 = X is M; 1 / 2 = Nesterov, X = G + beta M with G in float32 / bf16.
  auto run = [&](auto wtype, auto gmode) {
    using WT = decltype(wtype);
    constexpr int GM = decltype(gmode)::value;
    using GT = std::integral_constant<bool, GM == 2>;
    float lm[kChunks][4], lw[kChunks][4];
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      int64_t off = 0;
      int cnt = 0, i0 = 0, j0 = 0;
      if (v < cm.total) cm.piece(v, off, cnt, i0, j0);
      float lg[4] = {0.f, 0.f, 0.f, 0.f};
      if (cnt == 4 && cm.vec_ok) {
        ld_vec4<F32>(Mb, off, lm[k]);
        ld_vec4<WT>(Wb, off, lw[k]);
        if constexpr (GM != 0) ld_vec4<GT>(Gb, off, lg);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lm[k][u] = u < cnt ? ld_elem<F32>(Mb, off + u) : 0.f;
          lw[k][u] = u < cnt ? ld_elem<WT>(Wb, off + u) : 0.f;
          if constexpr (GM != 0) lg[u] = u < cnt ? ld_elem<GT>(Gb, off + u) : 0.f;
        }
      }
      if constexpr (GM != 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) lm[k][u] = fmaf(beta, lm[k][u], lg[u]);
      }
    }
    // Stage X (M, or G + beta M) in oriented order.
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      if (v >= cm.total) continue;
      int64_t off;
      int cnt, i0, j0;
      cm.piece(v, off, cnt, i0, j0);
      if (!cm.tr && cnt == 4) {
        *reinterpret_cast<f32x4_t*>(&st[i0][j0]) = f32x4_t{lm[k][0], lm[k][1], lm[k][2], lm[k][3]};
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u >= cnt) break;
          int i, j;
          cm.pos(i0, j0, u, i, j);
          st[i][j] = lm[k][u];
        }
      }
    }
    __syncthreads();

    // Qs as the A operand; the contraction index runs over rows rho of X.
    bf16x8_t qh[2], ql[2];
    float qf[BF16 ? 1 : 16];
    if constexpr (BF16) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float v = qs[col][rho(8 * g + t, h)];
          const __bf16 hi = (__bf16)v;
          qh[g][t] = hi;
          ql[g][t] = (__bf16)(v - (float)hi);
        }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) qf[r] = qs[col][rho(r, h)];
    }
    // O = Qs X per 32-column tile; X read in the column layout, O written
    // back over it (each wave owns its tiles).
#pragma unroll
    for (int q = 0; q < kTilesPerWave; ++q) {
      const int t = wave + kWaves * q;
      if (t * 32 >= cm.cw) break;
      const int j = t * 32 + col;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = st[rho(r, h)][j];  // rows >= m and columns >= cw are zero
      f32x16_t o = {};
      if constexpr (BF16) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          if (g == 1 && m <= 16) break;
          uint32_t hw[4], lw2[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x0 = x[8 * g + 2 * u], x1 = x[8 * g + 2 * u + 1];
            hw[u] = pack_bf16x2(x0, x1);
            lw2[u] = pack_bf16x2(x0 - bf16_lo(hw[u]), x1 - bf16_hi(hw[u]));
          }
          const bf16x8_t xh = as_bf16x8(hw[0], hw[1], hw[2], hw[3]);
          const bf16x8_t xl = as_bf16x8(lw2[0], lw2[1], lw2[2], lw2[3]);
          o = mfma_bf16(qh[g], xh, o);
          o = mfma_bf16(qh[g], xl, o);
          o = mfma_bf16(ql[g], xh, o);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (rho(r, 0) >= m) continue;
          o = mfma_f32(qf[r], x[r], o);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) st[rho(r, h)][j] = o[r];
    }
    __syncthreads();

    // W <- W - decay W - lr f O in storage order.
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      if (v >= cm.total) continue;
      int64_t off;
      int cnt, i0, j0;
      cm.piece(v, off, cnt, i0, j0);
      float w[4];
      if (!cm.tr && cnt == 4) {
        const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(&st[i0][j0]);
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = lw[k][u] - decay * lw[k][u] - lrf * o4[u];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int i = 0, j = 0;
          if (u < cnt) cm.pos(i0, j0, u, i, j);
          w[u] = lw[k][u] - decay * lw[k][u] - lrf * (u < cnt ? st[i][j] : 0.f);
        }
      }
      if (cnt == 4 && cm.vec_ok) {
        st_vec4<WT>(Wb, off, w);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (u < cnt) st_elem<WT>(Wb, off + u, w[u]);
      }
    }
  };
  // Rows >= m and columns >= cw of the staging block read as zero.
  zero_unfilled(st, m, cm.cw, tid);
  using G0 = std::integral_constant<int, 0>;
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  if constexpr (!NEST) {
    if (d.pdtype) run(B16{}, G0{});
    else run(F32{}, G0{});
  } else if (d.gdtype) {
    if (d.pdtype) run(B16{}, G2{});
    else run(F32{}, G2{});
  } else {
    if (d.pdtype) run(B16{}, G1{});
    else run(F32{}, G1{});
  }
}

}  // namespace

hipError_t launch_skinny_gram(const SkinnyLaunch& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, a.count);
  if (a.bf16) hipLaunchKernelGGL(k_skinny_gram<true>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_skinny_gram<false>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_skinny_apply(const SkinnyLaunch& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, a.count);
  if (a.nesterov) {
    if (a.bf16) hipLaunchKernelGGL((k_skinny_apply<true, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_skinny_apply<false, true>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.bf16) hipLaunchKernelGGL((k_skinny_apply<true, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_skinny_apply<false, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muon
