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
// Three launches per step, each over every skinny bucket of the plan (a
// workgroup finds its bucket in a table by its flat item or slice index):
//   k_skinny_gram   momentum M <- beta M + G (stored), and per 256-column
//                   chunk the Gram partial of X0 (M, or G + beta M with
//                   Nesterov momentum) on the matrix cores (split-K over the
//                   long dimension);
//   k_skinny_poly   per slice: the sum of the partials, s = 1/(||X0||_F +
//                   eps) from its trace, the k-round recurrence from
//                   A0 = s^2 (the sum) in float64, Qs = s Q;
//   k_skinny_apply  O = Qs X0 (matrix cores), W <- W - decay W - lr f O.
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

// Zero the part of a staging block of `rows` rows that a chunk does not
// fill: rows m .. rows-1, and columns >= cw of the rows below m.
__device__ __forceinline__ void zero_unfilled(float (*st)[kStride], int rows, int m, int cw, int tid) {
  for (int e = tid; e < (rows - m) * kCols; e += kThreads) st[m + e / kCols][e % kCols] = 0.f;
  if (cw < kCols) {
    const int w = kCols - cw;
    for (int e = tid; e < m * w; e += kThreads) st[e / w][cw + e % w] = 0.f;
  }
}

// The bucket of a flat (slice, chunk) item, or of a flat slice (by_slice):
// the last bucket whose first item (slice) is at or before it, by binary
// search over the table (uniform over the workgroup).
__device__ __forceinline__ int bucket_of(const SkinnyLaunch& a, int idx, bool by_slice) {
  int lo = 0, hi = a.n_buckets - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((by_slice ? a.buckets[mid].slice0 : a.buckets[mid].item0) <= idx) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// The bucket itself (the first one from the launch arguments).
__device__ __forceinline__ SkinnyBucket find_bucket(const SkinnyLaunch& a, int idx, bool by_slice) {
  if (a.n_buckets == 1) return a.b0;
  return a.buckets[bucket_of(a, idx, by_slice)];
}
// Slice and chunk of this workgroup in the Gram and apply launches: a plan
// with one skinny shape launches a (chunk, slice) grid, several shapes one
// flat grid over all items.
__device__ __forceinline__ SkinnyBucket chunk_of(const SkinnyLaunch& a, int& z, int& chunk) {
  if (gridDim.y > 1 || a.n_buckets == 1) {
    z = blockIdx.y;
    chunk = blockIdx.x;
    return a.b0;
  }
  const int item = blockIdx.x;
  const SkinnyBucket bk = find_bucket(a, item, false);
  const int r = item - bk.item0;
  z = r / bk.n_chunks;
  chunk = r - z * bk.n_chunks;
  return bk;
}

// ------------------------------------------------------------------ gram
// LDS of k_skinny_gram.  bf16 mode: the m staged rows as two bf16 planes,
// hi = bf16(x) and lo = bf16(x - hi), each with one more row of zeros (row
// m) that stands in for the padding rows m .. 31 of the products.  fp32 mode: the m staged float32 rows,
// or the waves' m x m float64 partials that reuse them, whichever is larger.
// Holding only m rows (not 32) lets more workgroups share a CU, so one
// workgroup's arithmetic overlaps another's memory traffic.
constexpr int kBStride = kCols + 8;  // bf16 plane row stride (elements; rows stay 16-byte aligned)
inline size_t skinny_gram_lds(int m, bool bf16) {
  if (bf16) return (size_t)2 * (m + 1) * kBStride * sizeof(uint16_t);
  const size_t stage = (size_t)m * kStride * sizeof(float);
  const size_t red = (size_t)kWaves * m * m * sizeof(double);
  return stage > red ? stage : red;
}

// Position of (i, j), i <= j, in an m x m upper triangle packed row by row.
__device__ __forceinline__ int tri_index(int i, int j, int m) { return i * m - (i * (i - 1)) / 2 + (j - i); }

// One 256-column chunk of slice z: M <- beta M + G (stored) and the chunk's
// Gram partial of X0 (M, or G + beta M with Nesterov momentum), stored as its
// packed upper triangle in float64.  (The slice's sum of squares is the
// trace of the summed partials.)  lds: skinny_gram_lds(m, BF16) bytes.
template <bool BF16>
__device__ __forceinline__ void gram_chunk(const SkinnyLaunch& a, const SkinnyBucket& bk, const DevScalars& S, int z,
                                           int chunk, float* lds) {
  float (*st)[kStride] = reinterpret_cast<float (*)[kStride]>(lds);         // fp32 mode: rows 0 .. m-1
  uint16_t (*H)[kBStride] = reinterpret_cast<uint16_t (*)[kBStride]>(lds);  // bf16 mode: hi plane
  const DevMat d = bk.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float beta = S.beta;
  const bool nesterov = S.nesterov != 0;
  const int m = bk.m, n = bk.n;
  uint16_t (*L)[kBStride] = H + m + 1;                                       // bf16 mode: lo plane
  const int tid = threadIdx.x, lane = tid & 63;
  // The wave index is uniform over the wave; saying so keeps branches on it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  ChunkMap cm;
  cm.init(m, n, chunk * kCols, min(kCols, n - chunk * kCols), d.transposed != 0, d.slice_off);
  char* const Mb = reinterpret_cast<char*>(pe.m + d.slice_off);
  const char* const Gb = static_cast<const char*>(pe.g) + d.slice_off * (d.gdtype ? 2 : 4);

  // bf16 mode, slice stored [m, n] with n % 4 == 0: each wave stages only
  // its own 64 columns (coalesced 16-byte pieces, four rows of 256 bytes per
  // load instruction), so its products need no barrier.
  const bool direct = BF16 && !cm.tr && cm.vec_ok;
  auto pass_direct = [&](auto gtype) {
    using GT = decltype(gtype);
    const int cb = wave * 64;
    float lm[kChunks][4], lg[kChunks][4];
    // Every piece is loaded, those outside the slice from the nearest piece
    // inside it (their values are not used): with no guard around a load,
    // the loads of all pieces are in flight together.  (cw is a multiple of
    // 4 on this path.)
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = lane + 64 * k, row = min(v >> 4, m - 1), cc = min(cb + 4 * (v & 15), cm.cw - 4);
      const int64_t off = (int64_t)row * n + cm.c0 + cc;
      ld_vec4<F32>(Mb, off, lm[k]);
      ld_vec4<GT>(Gb, off, lg[k]);
    }
    if (lane < 16) {
      *reinterpret_cast<u32x2_t*>(&H[m][cb + 4 * lane]) = u32x2_t{0u, 0u};
      *reinterpret_cast<u32x2_t*>(&L[m][cb + 4 * lane]) = u32x2_t{0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = lane + 64 * k, row = v >> 4, cc = cb + 4 * (v & 15);
      if (row >= m) continue;
      u32x2_t hv = {0u, 0u}, lv = {0u, 0u};
      if (cc < cm.cw) {
        float mn[4], xs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          mn[u] = fmaf(beta, lm[k][u], lg[k][u]);
          xs[u] = nesterov ? fmaf(beta, mn[u], lg[k][u]) : mn[u];
        }
        st_vec4<F32>(Mb, (int64_t)row * n + cm.c0 + cc, mn);
        hv = u32x2_t{pack_bf16x2(xs[0], xs[1]), pack_bf16x2(xs[2], xs[3])};
        lv = u32x2_t{pack_bf16x2(xs[0] - bf16_lo(hv.x), xs[1] - bf16_hi(hv.x)),
                     pack_bf16x2(xs[2] - bf16_lo(hv.y), xs[3] - bf16_hi(hv.y))};
      }
      *reinterpret_cast<u32x2_t*>(&H[row][cc]) = hv;
      *reinterpret_cast<u32x2_t*>(&L[row][cc]) = lv;
    }
    // This wave reads back only what it wrote; LDS accesses of one wave are
    // performed in order, so no barrier is needed, only that the compiler
    // keeps the order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (direct) {
    if (d.gdtype) pass_direct(B16{});
    else pass_direct(F32{});
  }

  // Columns >= cw of the staged rows, and the zero row m, read as zero.
  if constexpr (BF16) {
    if (!direct) for (int e = tid; e < kCols; e += kThreads) {
      H[m][e] = 0;
      L[m][e] = 0;
    }
    if (!direct && cm.cw < kCols) {
      const int w = kCols - cm.cw;
      for (int e = tid; e < m * w; e += kThreads) {
        H[e / w][cm.cw + e % w] = 0;
        L[e / w][cm.cw + e % w] = 0;
      }
    }
  } else {
    zero_unfilled(st, m, m, cm.cw, tid);
  }

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
      if constexpr (BF16) {
        if (!cm.tr && cnt == 4) {
          const uint32_t h0 = pack_bf16x2(xs[0], xs[1]), h1 = pack_bf16x2(xs[2], xs[3]);
          const uint32_t l0 = pack_bf16x2(xs[0] - bf16_lo(h0), xs[1] - bf16_hi(h0));
          const uint32_t l1 = pack_bf16x2(xs[2] - bf16_lo(h1), xs[3] - bf16_hi(h1));
          *reinterpret_cast<u32x2_t*>(&H[i0][j0]) = u32x2_t{h0, h1};
          *reinterpret_cast<u32x2_t*>(&L[i0][j0]) = u32x2_t{l0, l1};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (u >= cnt) break;
            int i, j;
            cm.pos(i0, j0, u, i, j);
            const uint16_t h = to_bf16(xs[u]);
            H[i][j] = h;
            L[i][j] = to_bf16(xs[u] - from_bf16(h));
          }
        }
      } else {
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
    }
  };
  if (!direct) {
    if (d.gdtype) pass(B16{});
    else pass(F32{});
    __syncthreads();
  }

  const int nt = m * (m + 1) / 2;
  double* const out = bk.gram_parts + ((int64_t)z * bk.n_chunks + chunk) * nt;
  if constexpr (BF16) {
    // Wave w multiplies its own 64 columns for the upper 16 x 16 tiles
    // (0, 0), (0, 16) and (16, 16) (only the first for m <= 16).  16x16x32
    // bf16 products (lane l: row l % 16 of the tile's A rows and of its B
    // rows, k = 8 (l / 16) .. + 7 of each 32-column step; result rows
    // 4 (l / 16) + r, column l % 16) accumulate hi hi + hi lo + lo hi + lo lo,
    // about float32 accuracy, in float32 per 32-column step and in float64
    // across steps; the four waves' sums are then added in wave order through
    // LDS, so the partial's rounding does not grow with the chunk width.
    // Rows >= m read the zero row m; columns >= cw are zero in the planes.
    const int li = lane & 15, kg = lane >> 4;
    const int ntile = m > 16 ? 3 : 1;
    auto rd = [](const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); };
    double accd[3][4];
#pragma unroll
    for (int tl = 0; tl < 3; ++tl) {
#pragma unroll
      for (int r = 0; r < 4; ++r) accd[tl][r] = 0.0;
      if (tl >= ntile) continue;
      const int ti = tl == 2 ? 16 : 0, tj = tl == 0 ? 0 : 16;
      const int rac = min(ti + li, m), rbc = min(tj + li, m);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = wave * 64 + t * 32 + kg * 8;
        const bf16x8_t ah = rd(&H[rac][c]), al = rd(&L[rac][c]);
        const bf16x8_t bh = ti == tj ? ah : rd(&H[rbc][c]), bl = ti == tj ? al : rd(&L[rbc][c]);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bl, acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) accd[tl][r] += (double)acc[r];
      }
    }
    __syncthreads();  // every wave is done with the planes, which now hold the sums
    double* const red = reinterpret_cast<double*>(lds);  // [4][nt]
#pragma unroll
    for (int tl = 0; tl < 3; ++tl) {
      if (tl >= ntile) continue;
      const int ti = tl == 2 ? 16 : 0, tj = tl == 0 ? 0 : 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti + 4 * kg + r, j = tj + li;
        if (i <= j && j < m) red[wave * nt + tri_index(i, j, m)] = accd[tl][r];
      }
    }
    __syncthreads();
    for (int e = tid; e < nt; e += kThreads) out[e] = ((red[e] + red[nt + e]) + red[2 * nt + e]) + red[3 * nt + e];
  } else {
    // fp32: lane l holds row l % 32 and both operands are the same rows; wave
    // w takes 32-column tiles w, w + 4, ...  Each tile is accumulated in
    // float32 on the matrix cores and added into a float64 running sum; the
    // four waves' partials are added through LDS.
    double* red = reinterpret_cast<double*>(lds);
    double accd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) accd[r] = 0.0;
    const int row = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int q = 0; q < kTilesPerWave; ++q) {
      const int t = wave + kWaves * q;
      if (t * 32 >= cm.cw) break;
      f32x16_t acc = {};
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        const float x = row < m ? st[row][t * 32 + 2 * s2 + kh] : 0.f;
        acc = mfma_f32(x, x, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) accd[r] += (double)acc[r];
    }
    // Output layout: lane l, register r -> row rho(r, l / 32), column l % 32.
    __syncthreads();  // every wave is done reading the staging block
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = rho(r, kh);
      if (i < m && row < m) red[(wave * m + i) * m + row] = accd[r];
    }
    __syncthreads();
    for (int e = tid; e < m * m; e += kThreads) {
      const int i = e / m, j = e - i * m;
      if (i > j) continue;
      double sum = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += red[w * m * m + e];
      out[tri_index(i, j, m)] = sum;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void k_skinny_gram(SkinnyLaunch a) {
  extern __shared__ __attribute__((aligned(16))) float gram_lds[];
  // The step's first kernel: scalars by value, written out for the later kernels.
  const DevScalars S = a.sc_out ? a.sv : *a.sc;
  if (a.sc_out && blockIdx.x == 0 && threadIdx.x == 0) *a.sc_out = a.sv;
  int z, chunk;
  const SkinnyBucket bk = chunk_of(a, z, chunk);
  gram_chunk<BF16>(a, bk, S, z, chunk, gram_lds);
}

// ------------------------------------------------------------------ poly
// Per slice: the sum G of the Gram partials, s = 1/(||X||_F + eps) from its
// trace, then the rounds in the m x m Gram space from A0 = s^2 G
// (A_{t+1} = P_t^2 A_t, Q = P_{k-1} ... P_0), all in float64, and finally
// s Q as float32.  The first round works on G itself with s^2 taken into
// its coefficients, so A0 is never formed.  Products
// run on the float64 matrix cores: each of the four waves owns one 16 x 16
// tile of a 32 x 32 result (16x16x4 float64 instruction: lane l supplies
// X[l % 16][l / 16] and Y[l / 16][l % 16] of each 4-wide k step and receives
// rows l / 16 + 4 r, r = 0..3, of column l % 16).  Everything outside the
// leading m x m block stays zero, so k steps past m (KQ = ceil(m / 4) is a
// template parameter, which keeps each product one straight run of
// instructions) and tiles past m are skipped: they would add exact zeros.
// A and Q are double-buffered, so a round needs three barriers.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef double f64x2_t __attribute__((ext_vector_type(2)));
constexpr int kPolyLd = 33;                                                  // row stride (doubles)
constexpr int kPolyLds = 6 * 32 * kPolyLd * (int)sizeof(double);  // A[2], Q[2], P and S
typedef double PolyRow[kPolyLd];

template <int KQ>
__device__ __forceinline__ void poly_slice(const SkinnyLaunch& a, const SkinnyBucket& bk, const DevScalars& Sc, int z,
                                           double* lds) {
  PolyRow* const base = reinterpret_cast<PolyRow*>(lds);
  PolyRow* const P = base + 128;
  PolyRow* const S = base + 160;
  auto Abuf = [&](int i) { return base + 32 * i; };
  auto Qbuf = [&](int i) { return base + 64 + 32 * i; };
  const int m = bk.m, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double ca = Sc.a, cb = Sc.b, cc = Sc.c;
  const int ns = Sc.ns_steps;
  const int nt = m * (m + 1) / 2;
  const int nch = bk.n_chunks;

  // Gram sums over the packed upper triangles, each entry summed in chunk
  // order.  Thread t takes the entry pairs (2 p, 2 p + 1), p = t + 256 k
  // (kPairs = 2 covers m <= 32): one 16-byte load per chunk where nt is even
  // (every pair then starts on a 16-byte boundary), two 8-byte loads
  // otherwise.  The loads of kBatch chunks are in flight together (all 40 of
  // n = 10240 in one batch where the registers allow), and the LDS is
  // cleared while the first batch is on its way.
  constexpr int kPairs = KQ <= 7 ? 1 : 2, kBatch = kPairs == 1 ? 40 : 20;
  const double* parts = bk.gram_parts + (int64_t)z * nch * nt;
  const bool even = (nt & 1) == 0;
  double sum[kPairs][2];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) sum[k][0] = sum[k][1] = 0.0;
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    f64x2_t part[kPairs][kBatch];
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int e0 = 2 * (tid + kThreads * k);
      if (e0 >= nt) continue;
      const bool two = e0 + 1 < nt;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = c0 + u < nch ? c0 + u : nch - 1;
        const double* q = parts + (int64_t)c * nt + e0;
        if (even) {
          part[k][u] = *reinterpret_cast<const MUON_GLOBAL f64x2_t*>(as_global(q));
        } else {
          part[k][u].x = *reinterpret_cast<const MUON_GLOBAL double*>(as_global(q));
          part[k][u].y = two ? *reinterpret_cast<const MUON_GLOBAL double*>(as_global(q + 1)) : 0.0;
        }
      }
    }
    if (c0 == 0)
      for (int e = tid; e < 6 * 32 * kPolyLd; e += kThreads) lds[e] = 0.0;
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      if (2 * (tid + kThreads * k) >= nt) continue;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const bool in = c0 + u < nch;
        sum[k][0] += in ? part[k][u].x : 0.0;
        sum[k][1] += in ? part[k][u].y : 0.0;
      }
    }
  }
  __syncthreads();
  // The summed Gram matrix G, both triangles, and Q = I.
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int e0 = 2 * (tid + kThreads * k);
    if (e0 >= nt) continue;
    int i = 0, r = e0;
    while (r >= m - i) {
      r -= m - i;
      ++i;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (e0 + h >= nt) break;
      if (h == 1 && ++r >= m - i) {  // the pair's second entry opens the next row
        r = 0;
        ++i;
      }
      Abuf(0)[i][i + r] = sum[k][h];
      Abuf(0)[i + r][i] = sum[k][h];
    }
  }
  for (int e = tid; e < m; e += kThreads) Qbuf(0)[e][e] = 1.0;
  __syncthreads();
  // Sum of squares of X0 = trace of G, summed by every thread in row order;
  // s = 1 / (||X0||_F + eps).  A0 = s^2 G is never formed: the first round
  // takes s^2 into its coefficients and into A1.
  double tr = 0.0;
  for (int i = 0; i < m; ++i) tr += Abuf(0)[i][i];
  const double s = 1.0 / (sqrt(tr) + (double)Sc.eps);
  if (tid == 0 && !isfinite(tr)) atomicOr(a.err, kErrNonFinite);
  const double s2 = s * s;

  const int ti = 16 * (wave >> 1), tj = 16 * (wave & 1);
  const int li = lane & 15, lk = lane >> 4;
  const bool live = ti < m && tj < m;  // this wave's tile has entries inside m x m
  // One tile of X Y: the operands of the k steps are read from LDS first,
  // then the products run in two independent chains (even and odd k steps).
  auto prod = [&](const PolyRow* X, const PolyRow* Y) {
    double xv[KQ], yv[KQ];
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      xv[q] = X[ti + li][4 * q + lk];
      yv[q] = Y[4 * q + lk][tj + li];
    }
    f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < KQ; q += 2) {
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[q], yv[q], acc0, 0, 0, 0);
      if (q + 1 < KQ) acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[q + 1], yv[q + 1], acc1, 0, 0, 0);
    }
    // Every operand read is issued before the first product, so the LDS
    // latency is paid once per tile rather than once per k step.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KQ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KQ, 0);
    return acc0 + acc1;
  };
  int cur = 0;
  for (int it = 0; it < ns; ++it) {
    const bool more = it + 1 < ns;
    PolyRow* const Ac = Abuf(cur);
    // Round 0 holds G = A0 / s^2: P = a I + (b s^2) G + (c s^4) G^2 and
    // A1 = s^2 P^2 G.
    const double kb = it == 0 ? cb * s2 : cb, kc = it == 0 ? cc * (s2 * s2) : cc, ka = it == 0 ? s2 : 1.0;
    // P = a I + b A + c A^2 (the entries of A read ahead of the product)
    if (live) {
      double av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = Ac[ti + lk + 4 * r][tj + li];
      const f64x4_t t = prod(Ac, Ac);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti + lk + 4 * r, j = tj + li;
        P[i][j] = kb * av[r] + kc * t[r] + ((i == j && i < m) ? ca : 0.0);
      }
    }
    __syncthreads();
    // Q' = P Q and, unless this is the last round, S = P P
    if (live) {
      const f64x4_t q = prod(P, Qbuf(cur));
      PolyRow* const Qn = Qbuf(cur ^ 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) Qn[ti + lk + 4 * r][tj + li] = q[r];
      if (more) {
        const f64x4_t sp = prod(P, P);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[ti + lk + 4 * r][tj + li] = sp[r];
      }
    }
    __syncthreads();
    if (more) {
      // A' = S A
      if (live) {
        const f64x4_t t = prod(S, Ac);
        PolyRow* const An = Abuf(cur ^ 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) An[ti + lk + 4 * r][tj + li] = ka * t[r];
      }
      __syncthreads();
    }
    cur ^= 1;
  }
  PolyRow* const Qf = Qbuf(cur);
  for (int e = tid; e < 1024; e += kThreads) bk.qs[(int64_t)z * 1024 + e] = (float)(s * Qf[e >> 5][e & 31]);
}

template <int KQ>
__global__ __launch_bounds__(kThreads) void k_skinny_poly(SkinnyLaunch a) {
  __shared__ double poly_lds[kPolyLds / sizeof(double)];
  const int slice = blockIdx.x;
  const SkinnyBucket bk = find_bucket(a, slice, true);
  poly_slice<KQ>(a, bk, *a.sc, slice - bk.slice0, poly_lds);
}

// ------------------------------------------------------------------ apply
// O = Qs X0 per 256-column chunk, then W <- W - decay W - lr f O.  Wave w
// takes columns [64 w, 64 w + 64) of the chunk; lane l owns the 4-column
// piece at 4 (l % 16) of them, rows R (l / 16) + q, q < R, of X0
// (R = 2 ceil(m / 8), so 4 R >= m) and rows 16 t + 4 (l / 16) + r of O.  16x16x4 float32
// products (lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// receives rows 4 (l / 16) + r of column l % 16): product (t, u) of k step q
// takes the contraction indices q, R + q, 2 R + q, 3 R + q, multiplies rows
// 16 t .. + 15 of Qs by element u of every lane's X0 piece, so its column j
// is column 4 j + u of the wave's 64, and the result lands in the lanes that
// hold the matching W piece.  A lane's Qs operands are then R consecutive
// entries of a row, read as 8-byte pieces.  Operands and accumulation are
// float32 in both modes.  The Qs operands and X0 are loaded before W, so the
// products start while the W loads are still in flight.  RM, the largest R
// of the launch, sizes the registers; R itself depends only on the slice.
// Two forms share this arithmetic, so a slice gives the same bits whichever
// way it is stored: slices stored [m, n] with n % 4 == 0 read their pieces
// straight from memory (no LDS, no barrier); the others are turned around in
// LDS first.

__device__ __forceinline__ int apply_rows(int m) { return 2 * ((m + 7) >> 3); }
template <int RM>
constexpr int apply_tiles() { return RM > 4 ? 2 : 1; }

// Qs operands: Qs[16 t + l % 16][R (l / 16) + q] (zero outside m x m).
template <int RM>
__device__ __forceinline__ void load_qs_operands(const float* Q, int p, int g, int R, int nt,
                                                 float (&qa)[apply_tiles<RM>()][RM]) {
#pragma unroll
  for (int t = 0; t < apply_tiles<RM>(); ++t)
#pragma unroll
    for (int h = 0; h < RM / 2; ++h) {
      f32x2_t v = {0.f, 0.f};
      if (t < nt && 2 * h < R) v = *reinterpret_cast<const MUON_GLOBAL f32x2_t*>(as_global(Q + (16 * t + p) * 32 + R * g + 2 * h));
      qa[t][2 * h] = v.x;
      qa[t][2 * h + 1] = v.y;
    }
}
template <int RM>
__device__ __forceinline__ void apply_products(const f32x4_t (&x)[RM], const float (&qa)[apply_tiles<RM>()][RM], int R,
                                               int nt, f32x4_t (&acc)[apply_tiles<RM>()][4]) {
#pragma unroll
  for (int t = 0; t < apply_tiles<RM>(); ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < RM; ++q) {
    if (q >= R) break;
#pragma unroll
    for (int t = 0; t < apply_tiles<RM>(); ++t) {
      if (t >= nt) break;
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][q], x[q][u], acc[t][u], 0, 0, 0);
    }
  }
}
// The update of one element: (W - decay W) - lr f O.
__device__ __forceinline__ float w_update(float w, float decay, float lrf, float o) {
  return fmaf(-lrf, o, fmaf(-decay, w, w));
}

// Direct form (slice stored [m, n], n % 4 == 0: every 4-column piece lies
// whole inside or outside the slice and is 16-byte aligned).
template <int RM, bool NEST>
__device__ __forceinline__ void apply_direct(const SkinnyLaunch& a, const SkinnyBucket& bk, const DevScalars& S, int z,
                                             int chunk) {
  const DevMat d = bk.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const int m = bk.m, n = bk.n;
  const float lrf = S.lr * update_factor(S.scale_mode, m, n, 0), decay = S.decay, beta = S.beta;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = lane & 15, g = lane >> 4;
  const int c = chunk * kCols + wave * 64 + 4 * p;  // first column of this lane's piece
  const bool in = c < n;
  const int R = apply_rows(m), nt = (m + 15) >> 4;
  constexpr int NT = apply_tiles<RM>();
  const float* const Mb = pe.m + d.slice_off;
  char* const Wb = static_cast<char*>(pe.w) + d.slice_off * (d.pdtype ? 2 : 4);

  // Every load first: the Qs operands, the X0 pieces, then the W pieces of
  // the lane's O rows.  X0 is loaded without guards, pieces outside the
  // slice from the nearest piece inside it (n is a multiple of 4 on this
  // path): a guard around a load makes the compiler wait for it at once.
  // The rows past the slice are zeroed before the products; a lane past the
  // slice's end only computes columns it does not store.
  float qa[NT][RM];
  load_qs_operands<RM>(bk.qs + (int64_t)z * 1024, p, g, R, nt, qa);
  f32x4_t x[RM];
#pragma unroll
  for (int q = 0; q < RM; ++q) {
    const int row = min(R * g + q, m - 1);
    x[q] = *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(Mb + (int64_t)row * n + (in ? c : n - 4)));
  }
  // Nesterov momentum: G at the same pieces, unguarded too, as its stored
  // bits (this kernel never writes G), converted where it is used.
  u32x4_t graw[NEST ? RM : 1];
  if constexpr (NEST) {
    const char* const Gb = static_cast<const char*>(pe.g) + d.slice_off * (d.gdtype ? 2 : 4);
    if (d.gdtype) {
#pragma unroll
      for (int q = 0; q < RM; ++q) {
        const int row = min(R * g + q, m - 1);
        const u32x2_t b = *reinterpret_cast<const MUON_GLOBAL u32x2_t*>(as_global(Gb) + 2 * ((int64_t)row * n + (in ? c : n - 4)));
        graw[q] = u32x4_t{b.x, b.y, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int q = 0; q < RM; ++q) {
        const int row = min(R * g + q, m - 1);
        graw[q] = *reinterpret_cast<const MUON_GLOBAL u32x4_t*>(as_global(Gb) + 4 * ((int64_t)row * n + (in ? c : n - 4)));
      }
    }
  }
  // W likewise, in the type it is stored in, by a copy of the rest of the
  // function per W dtype, so that no guard or conversion sits next to a
  // load.  (A form that loaded a float32 W as integer words and stored it
  // as floats gave wrong results; loads and stores of one type do not.)
  auto w_pass = [&](auto b16_tag) {
    constexpr bool kB16 = decltype(b16_tag)::value;
    using Raw = typename std::conditional<kB16, u32x2_t, f32x4_t>::type;
    const int cl = in ? c : n - 4;  // n is a multiple of 4 on this path
    Raw wr[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = min(16 * t + 4 * g + r, m - 1);
        wr[t][r] = *reinterpret_cast<const MUON_GLOBAL Raw*>(as_global(Wb) + (kB16 ? 2 : 4) * ((int64_t)row * n + cl));
      }
#pragma unroll
    for (int q = 0; q < RM; ++q)
      if (q >= R || R * g + q >= m) x[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (NEST) {
#pragma unroll
      for (int q = 0; q < RM; ++q) {
        f32x4_t gq;
        if (d.gdtype) {
          gq = f32x4_t{bf16_lo(graw[q].x), bf16_hi(graw[q].x), bf16_lo(graw[q].y), bf16_hi(graw[q].y)};
        } else {
          gq = __builtin_bit_cast(f32x4_t, graw[q]);
        }
        if (q >= R || R * g + q >= m) gq = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) x[q][u] = fmaf(beta, x[q][u], gq[u]);
      }
    }
    f32x4_t acc[NT][4];
    apply_products<RM>(x, qa, R, nt, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * t + 4 * g + r;
        if (t >= nt || !in || row >= m) continue;
        float w[4];
        if constexpr (kB16) {
          w[0] = bf16_lo(wr[t][r].x);
          w[1] = bf16_hi(wr[t][r].x);
          w[2] = bf16_lo(wr[t][r].y);
          w[3] = bf16_hi(wr[t][r].y);
        } else {
          w[0] = wr[t][r].x;
          w[1] = wr[t][r].y;
          w[2] = wr[t][r].z;
          w[3] = wr[t][r].w;
        }
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = w_update(w[u], decay, lrf, acc[t][u][r]);
        if constexpr (kB16) st_vec4<B16>(Wb, (int64_t)row * n + c, o);
        else st_vec4<F32>(Wb, (int64_t)row * n + c, o);
      }
  };
  if (d.pdtype) w_pass(std::true_type{});
  else w_pass(std::false_type{});
}

// Staged form (any slice): the chunk's X0 is turned around in LDS, the
// products read their pieces from there and write O back over them, and W is
// updated in storage order.  lds: 32 staged rows (rows m .. 31 and columns
// past the chunk are zero).
template <int RM, bool NEST>
__device__ __forceinline__ void apply_chunk(const SkinnyLaunch& a, const SkinnyBucket& bk, const DevScalars& S, int z,
                                            int chunk, float* lds) {
  float (*st)[kStride] = reinterpret_cast<float (*)[kStride]>(lds);
  const DevMat d = bk.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float lr = S.lr, decay = S.decay, beta = S.beta;
  const int m = bk.m, n = bk.n;
  const float lrf = lr * update_factor(S.scale_mode, m, n, d.transposed);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  ChunkMap cm;
  cm.init(m, n, chunk * kCols, min(kCols, n - chunk * kCols), d.transposed != 0, d.slice_off);
  const char* const Mb = reinterpret_cast<const char*>(pe.m + d.slice_off);
  const char* const Gb = static_cast<const char*>(pe.g) + d.slice_off * (d.gdtype ? 2 : 4);
  char* const Wb = static_cast<char*>(pe.w) + d.slice_off * (d.pdtype ? 2 : 4);

  // gmode: 0 = G is not read; 1 / 2 = Nesterov, X = G + beta M with G in
  // float32 / bf16.
  auto run = [&](auto wtype, auto gmode) {
    using WT = decltype(wtype);
    constexpr int GM = decltype(gmode)::value;
    using GT = std::integral_constant<bool, GM == 2>;
    float lm[kChunks][4], lw[kChunks][4], lg[kChunks][4];
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int v = tid + kThreads * k;
      int64_t off = 0;
      int cnt = 0, i0 = 0, j0 = 0;
      if (v < cm.total) cm.piece(v, off, cnt, i0, j0);
      if (cnt == 4 && cm.vec_ok) {
        ld_vec4<F32>(Mb, off, lm[k]);
        ld_vec4<WT>(Wb, off, lw[k]);
        if constexpr (GM != 0) ld_vec4<GT>(Gb, off, lg[k]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lm[k][u] = u < cnt ? ld_elem<F32>(Mb, off + u) : 0.f;
          lw[k][u] = u < cnt ? ld_elem<WT>(Wb, off + u) : 0.f;
          if constexpr (GM != 0) lg[k][u] = u < cnt ? ld_elem<GT>(Gb, off + u) : 0.f;
        }
      }
    }
    if constexpr (NEST) {
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
#pragma unroll
        for (int u = 0; u < 4; ++u) lm[k][u] = fmaf(beta, lm[k][u], lg[k][u]);
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

    // The products on the wave's own 64 columns; O replaces X in place.
    {
      const int p = lane & 15, g = lane >> 4, c = wave * 64 + 4 * p;
      const int R = apply_rows(m), nt = (m + 15) >> 4;
      constexpr int NT = apply_tiles<RM>();
      float qa[NT][RM];
      load_qs_operands<RM>(bk.qs + (int64_t)z * 1024, p, g, R, nt, qa);
      f32x4_t x[RM];
#pragma unroll
      for (int q = 0; q < RM; ++q)
        x[q] = q < R ? *reinterpret_cast<const f32x4_t*>(&st[R * g + q][c]) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      f32x4_t acc[NT][4];
      apply_products<RM>(x, qa, R, nt, acc);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nt) break;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<f32x4_t*>(&st[16 * t + 4 * g + r][c]) =
              f32x4_t{acc[t][0][r], acc[t][1][r], acc[t][2][r], acc[t][3][r]};
      }
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
        for (int u = 0; u < 4; ++u) w[u] = w_update(lw[k][u], decay, lrf, o4[u]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int i = 0, j = 0;
          if (u < cnt) cm.pos(i0, j0, u, i, j);
          w[u] = w_update(lw[k][u], decay, lrf, u < cnt ? st[i][j] : 0.f);
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
  // Rows m .. 31, and columns >= cw of the staged rows, read as zero.
  zero_unfilled(st, 32, m, cm.cw, tid);
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

// NEST is chosen at launch from the plan, so the plain kernel carries no
// second code path.
template <int RM, bool NEST>
__global__ __launch_bounds__(kThreads) void k_skinny_apply(SkinnyLaunch a) {
  extern __shared__ __attribute__((aligned(16))) float apply_lds[];  // 32 staged rows
  int z, chunk;
  const SkinnyBucket bk = chunk_of(a, z, chunk);
  // The form depends only on the slice's own layout (uniform per workgroup).
  if (!bk.mats[z].transposed && (bk.n & 3) == 0) apply_direct<RM, NEST>(a, bk, *a.sc, z, chunk);
  else apply_chunk<RM, NEST>(a, bk, *a.sc, z, chunk, apply_lds);
}

}  // namespace

// One skinny shape: a (chunk, slice) grid; several: one flat grid over all items.
inline dim3 chunk_grid(const SkinnyLaunch& a) {
  return a.n_buckets == 1 ? dim3(a.b0.n_chunks, a.b0.count) : dim3(a.items);
}

hipError_t launch_skinny_gram(const SkinnyLaunch& a, hipStream_t s) {
  const dim3 grid = chunk_grid(a);
  const size_t lds = skinny_gram_lds(a.m_max, a.bf16 != 0);
  if (a.bf16) hipLaunchKernelGGL(k_skinny_gram<true>, grid, dim3(kThreads), lds, s, a);
  else hipLaunchKernelGGL(k_skinny_gram<false>, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_skinny_poly(const SkinnyLaunch& a, hipStream_t s) {
  // Buckets with a smaller m run the largest m's k steps over zero padding.
  const dim3 grid(a.slices), block(kThreads);
  switch ((a.m_max + 3) >> 2) {
    case 1: hipLaunchKernelGGL(k_skinny_poly<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_skinny_poly<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_skinny_poly<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_skinny_poly<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(k_skinny_poly<5>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(k_skinny_poly<6>, grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL(k_skinny_poly<7>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_skinny_poly<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_skinny_apply(const SkinnyLaunch& a, hipStream_t s) {
  const dim3 grid = chunk_grid(a);
  const size_t lds = (size_t)32 * kStride * sizeof(float);
  // RM = 2 ceil(m_max / 8): registers for the largest slice of the launch.
#define MUON_APPLY_CASE(RM)                                                                     \
  case RM:                                                                                      \
    if (a.nesterov) hipLaunchKernelGGL((k_skinny_apply<RM, true>), grid, dim3(kThreads), lds, s, a); \
    else hipLaunchKernelGGL((k_skinny_apply<RM, false>), grid, dim3(kThreads), lds, s, a);           \
    break;
  switch (2 * ((a.m_max + 7) >> 3)) {
    MUON_APPLY_CASE(2)
    MUON_APPLY_CASE(4)
    MUON_APPLY_CASE(6)
    MUON_APPLY_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MUON_APPLY_CASE
  return hipGetLastError();
}

}  // namespace muon
