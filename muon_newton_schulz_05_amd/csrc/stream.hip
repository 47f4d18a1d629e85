// stream.hip -- kernels of the streamed path (slices with m > 32).
//
// Per step and shape bucket:
//   momentum  M <- beta M + G, per-tile sums of squares, X0 = M (oriented) and
//             its transpose into the workspace          ("关于分布式Muon的想法整合及讨论"
//                                                        §1, §2, §6)
//   norm      s = 1 / (||M||_F + eps) from the tile sums, fixed order
//   k rounds  gram   A = X X^T          (s^2 folded in on the first round)
//             poly   P = b A + c A A
//             apply  X' = a X + P X     (s folded in on the first round;
//                                         the last round updates W instead)
// ("MindSpore HyperParallel X 盘古,Muon优化器实现6倍性能跃升", 三大性能挑战: the
// iteration is rounds of matrix products and additions.)
//
// Every product is C[i][j] = sum_k A[i][k] B[j][k] with both operands
// contiguous along k: X X^T reads X twice, A A reads the symmetric A twice,
// P X reads P and the transposed copy X^T that the previous round wrote.
// Workspace matrices are zero-padded to multiples of 128, so the products run
// on whole tiles and the padding stays exactly zero.
#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

// ------------------------------------------------------------------ prologue
__global__ void k_prologue(DevScalars* dst, DevScalars v) {
  if (threadIdx.x == 0) *dst = v;
}

// ------------------------------------------------------------------ momentum
// Four consecutive workspace entries of X (float32, or bf16 rounded to
// nearest even) in one store.
__device__ __forceinline__ void store_x4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(p)) = f32x4_t{a, b, c, d};
}
__device__ __forceinline__ void store_x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(p)) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

template <typename XT>
__global__ __launch_bounds__(256) void k_momentum(MomentumLaunch a) {
  __shared__ float tile[kMomTile][kMomTile + 1];
  __shared__ float wsum[4];
  const int z = blockIdx.y;
  const int tiles_n = (int)((a.n + kMomTile - 1) / kMomTile);
  const int ti = blockIdx.x / tiles_n, tj = blockIdx.x % tiles_n;
  const int64_t i0 = (int64_t)ti * kMomTile, j0 = (int64_t)tj * kMomTile;
  const DevMat d = a.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float beta = a.sc_out ? a.sv.beta : a.sc->beta;
  const bool nesterov = (a.sc_out ? a.sv.nesterov : a.sc->nesterov) != 0;
  if (a.sc_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.sc_out = a.sv;
  const int tid = threadIdx.x;

  // Load along the stored rows (coalesced), keep X0 in LDS in oriented order:
  // M_new, or G + beta M_new with Nesterov momentum.  A whole tile whose
  // stored rows start on 4-element boundaries moves 4 consecutive elements
  // per access (16 bytes of M); any other tile goes element by element.
  const int64_t len = d.transposed ? a.m : a.n;  // stored row length
  const bool whole = i0 + kMomTile <= a.m && j0 + kMomTile <= a.n && (len & 3) == 0 && (d.slice_off & 3) == 0;
  if (whole) {
    const int64_t s0 = d.transposed ? j0 : i0, c0 = d.transposed ? i0 : j0;  // stored tile origin
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sr = (tid >> 4) + 16 * q, sc = 4 * (tid & 15);
      const int64_t idx = d.slice_off + (s0 + sr) * len + c0 + sc;
      f32x4_t g;
      if (d.gdtype == 1) {
        const u32x2_t w = *reinterpret_cast<const MUON_GLOBAL u32x2_t*>(as_global(static_cast<const uint16_t*>(pe.g) + idx));
        g = f32x4_t{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
      } else {
        g = *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(static_cast<const float*>(pe.g) + idx));
      }
      MUON_GLOBAL f32x4_t* mp4 = reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(pe.m + idx));
      const f32x4_t m0 = *mp4;
      const f32x4_t mn{fmaf(beta, m0.x, g.x), fmaf(beta, m0.y, g.y), fmaf(beta, m0.z, g.z), fmaf(beta, m0.w, g.w)};
      *mp4 = mn;
      const f32x4_t v = nesterov ? f32x4_t{fmaf(beta, mn.x, g.x), fmaf(beta, mn.y, g.y), fmaf(beta, mn.z, g.z),
                                           fmaf(beta, mn.w, g.w)}
                                 : mn;
      if (d.transposed) {
        tile[sc + 0][sr] = v.x;
        tile[sc + 1][sr] = v.y;
        tile[sc + 2][sr] = v.z;
        tile[sc + 3][sr] = v.w;
      } else {
        tile[sr][sc + 0] = v.x;
        tile[sr][sc + 1] = v.y;
        tile[sr][sc + 2] = v.z;
        tile[sr][sc + 3] = v.w;
      }
    }
  } else {
    for (int q = 0; q < 16; ++q) {
      const int fast = tid & 63, slow = (tid >> 6) + 4 * q;
      const int ii = d.transposed ? fast : slow;
      const int jj = d.transposed ? slow : fast;
      const int64_t i = i0 + ii, j = j0 + jj;
      float v = 0.f;
      if (i < a.m && j < a.n) {
        const int64_t idx = d.slice_off + (d.transposed ? j * a.m + i : i * a.n + j);
        const float g = load_as_f32(pe.g, idx, d.gdtype);
        const float mn = fmaf(beta, pe.m[idx], g);
        pe.m[idx] = mn;
        v = nesterov ? fmaf(beta, mn, g) : mn;
      }
      tile[ii][jj] = v;
    }
  }
  __syncthreads();

  // Sum of squares in a fixed order over the oriented tile (entries outside
  // the slice are zero).
  float sq = 0.f;
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q;
    const float v = tile[e >> 6][e & 63];
    sq = fmaf(v, v, sq);
  }
  // X and X^T in 4-element pieces.  The workspace is padded to whole tiles
  // and entries outside the slice are zero in the tile, so whole pieces stay
  // inside the buffers and leave the padding zero.
  XT* x = static_cast<XT*>(a.x) + (int64_t)z * a.mp * a.np;
  XT* xt = static_cast<XT*>(a.xt) + (int64_t)z * a.mp * a.np;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 4) + 16 * q, c = 4 * (tid & 15);
    store_x4(x + (i0 + r) * a.np + j0 + c, tile[r][c], tile[r][c + 1], tile[r][c + 2], tile[r][c + 3]);
    store_x4(xt + (j0 + r) * a.mp + i0 + c, tile[c][r], tile[c + 1][r], tile[c + 2][r], tile[c + 3][r]);
  }
  sq = wave_sum(sq);
  if ((tid & 63) == 0) wsum[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) a.sq[(int64_t)z * a.km_tiles + blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// ------------------------------------------------------------------ norm
__global__ __launch_bounds__(256) void k_norm(NormLaunch a) {
  __shared__ double red[256];
  const int z = blockIdx.x;
  double s = 0.0;
  for (int t = threadIdx.x; t < a.km_tiles; t += 256) s += (double)a.sq[(int64_t)z * a.km_tiles + t];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double sc = 1.0 / (sqrt(red[0]) + (double)a.sc->eps);
    a.scale[2 * z] = (float)sc;
    a.scale[2 * z + 1] = (float)(sc * sc);
    // A non-finite momentum entry makes the sum non-finite; the update of
    // this slice is then not finite either, and the plan's error word says so.
    if (!isfinite(red[0])) atomicOr(a.err, kErrNonFinite);
  }
}

// ------------------------------------------------------------------ matrix-core helpers
__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ epilogues
struct GramEpi {
  float* a32;
  const float* scale;
  int64_t mp;
  __device__ void operator()(int z, int i0, int j, const float v[4]) const {
    const float s = scale ? scale[2 * z + 1] : 1.f;
    const int64_t zb = (int64_t)z * mp * mp;
#pragma unroll
    for (int u = 0; u < 4; ++u) a32[zb + (int64_t)(i0 + u) * mp + j] = s * v[u];
  }
};

struct PolyEpi {
  const float* a32;
  void* phi;
  uint16_t* plo;
  int p_f32;
  const DevScalars* sc;
  int64_t mp;
  __device__ void put(int64_t idx, float val) const {
    if (p_f32) {
      static_cast<float*>(phi)[idx] = val;
    } else {
      const uint16_t hi = to_bf16(val);
      static_cast<uint16_t*>(phi)[idx] = hi;
      if (plo) plo[idx] = to_bf16(val - from_bf16(hi));
    }
  }
  __device__ void operator()(int z, int i0, int j, const float v[4]) const {
    const float b = sc->b, c = sc->c;
    const int64_t zb = (int64_t)z * mp * mp;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t idx = zb + (int64_t)(i0 + u) * mp + j;
      put(idx, b * a32[idx] + c * v[u]);
    }
  }
};

template <typename XT>
struct ApplyEpi {
  const XT* x_old;
  XT* x_new;
  XT* xt_new;
  const float* scale;
  const DevScalars* sc;
  int64_t mp, np;
  __device__ void operator()(int z, int i0, int j, const float v[4]) const {
    const float s = scale ? scale[2 * z] : 1.f;
    const float a = sc->a;
    const int64_t zo = (int64_t)z * mp * np;
    XT out[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t idx = zo + (int64_t)(i0 + u) * np + j;
      const float val = s * fmaf(a, x_to_f32(x_old[idx]), v[u]);
      out[u] = cvt_x<XT>(val);
      x_new[idx] = out[u];
    }
    XT* t = xt_new + zo + (int64_t)j * mp + i0;
    if constexpr (sizeof(XT) == 2) {
      uint2 p;
      p.x = (uint32_t)out[0] | ((uint32_t)out[1] << 16);
      p.y = (uint32_t)out[2] | ((uint32_t)out[3] << 16);
      *reinterpret_cast<uint2*>(t) = p;
    } else {
      *reinterpret_cast<float4*>(t) = make_float4(out[0], out[1], out[2], out[3]);
    }
  }
};

template <typename XT>
struct FinalEpi {
  const XT* x_old;
  const float* scale;
  const DevScalars* sc;
  const DevMat* mats;
  const PtrEntry* ptrs;
  int64_t mp, np, m, n;
  __device__ void operator()(int z, int i0, int j, const float v[4]) const {
    const float s = scale ? scale[2 * z] : 1.f;
    const DevMat d = mats[z];
    const PtrEntry pe = ptrs[d.param];
    const float a = sc->a, decay = sc->decay;
    const float lrf = sc->lr * update_factor(sc->scale_mode, m, n, d.transposed);
    const int64_t zo = (int64_t)z * mp * np;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u;
      if (i < m && j < n) {
        const float val = s * fmaf(a, x_to_f32(x_old[zo + i * np + j]), v[u]);
        const int64_t idx = d.slice_off + (d.transposed ? (int64_t)j * m + i : i * n + j);
        const float w = load_as_f32(pe.w, idx, d.pdtype);
        store_from_f32(pe.w, idx, d.pdtype, w - decay * w - lrf * val);
      }
    }
  }
};

// ------------------------------------------------------------------ ns_steps = 0
__global__ __launch_bounds__(256) void k_update0(Update0Launch a) {
  const int z = blockIdx.y;
  const DevMat d = a.mats[z];
  const PtrEntry pe = a.ptrs[d.param];
  const float k = a.sc->lr * update_factor(a.sc->scale_mode, a.m, a.n, d.transposed) * a.scale[2 * z];
  const float decay = a.sc->decay, beta = a.sc->beta;
  const bool nesterov = a.sc->nesterov != 0;
  const int64_t total = a.m * a.n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t idx = d.slice_off + e;  // stored order; O and W share the layout
    const float w = load_as_f32(pe.w, idx, d.pdtype);
    const float x = nesterov ? fmaf(beta, pe.m[idx], load_as_f32(pe.g, idx, d.gdtype)) : pe.m[idx];
    store_from_f32(pe.w, idx, d.pdtype, w - decay * w - k * x);
  }
}

// ------------------------------------------------------------------ grouped products: shared parts
// The streamed products run grouped: each product phase of a round is one
// launch over every bucket of a group (the small buckets, padded m <= 256; or
// the others), and workgroup b belongs to the last bucket with
// t0[phase] <= b.  The tile grid of a bucket, and the split of each output
// entry's sum, depend on its shape alone, so fused and single-slice runs give
// the same bits.

// Ph: 0 gram (A = s2 X X^T), 1 poly (P = b A + c A A), 2 apply (X' = s (a X + P X)),
// 3 the last round's apply, which updates W.  PH: the tile grid of the phase.
template <int Ph>
constexpr int grid_phase() { return Ph == 3 ? 2 : Ph; }

template <int PH>
__device__ __forceinline__ const SmallBucket& find_bucket(const SmallArgs& g, int wg) {
  int lo = 0, hi = g.nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.buckets[mid].t0[PH] <= wg) lo = mid;
    else hi = mid - 1;
  }
  return g.buckets[lo];
}

// The round's ping-pong buffers, chosen without indexing a local array by a
// run-time value (which would put the bucket in scratch memory).
struct RoundBuffers {
  char *x_src, *x_dst, *xt_src, *xt_dst;
};
__device__ __forceinline__ RoundBuffers round_buffers(const SmallBucket& bk, int src) {
  return {src ? bk.x[1] : bk.x[0], src ? bk.x[0] : bk.x[1], src ? bk.xt[1] : bk.xt[0], src ? bk.xt[0] : bk.xt[1]};
}

// Operands of slice z: rows of A and of B, both contiguous along k, with
// row stride ld and contraction length K (the padded m or n).  The apply's
// P may come as a bf16 hi/lo pair (a, a2).
struct Operands {
  const char *a, *a2, *b;
  int64_t ld, K;
};
template <typename T, int Ph>
__device__ __forceinline__ Operands slice_operands(const SmallBucket& bk, const RoundBuffers& rb, int z) {
  constexpr int ES = (int)sizeof(T);
  Operands o{};
  if constexpr (Ph == 0) {
    o.a = o.b = rb.x_src + (int64_t)z * bk.mp * bk.np * ES;
    o.ld = o.K = bk.np;
  } else if constexpr (Ph == 1) {
    o.a = o.b = reinterpret_cast<const char*>(bk.a32 + (int64_t)z * bk.mp * bk.mp);
    o.ld = o.K = bk.mp;
  } else {
    o.a = bk.phi + (int64_t)z * bk.mp * bk.mp * ES;
    if (bk.plo) o.a2 = reinterpret_cast<const char*>(bk.plo + (int64_t)z * bk.mp * bk.mp);
    o.b = rb.xt_src + (int64_t)z * bk.np * bk.mp * ES;
    o.ld = o.K = bk.mp;
  }
  return o;
}

// The phase's epilogue for 4 consecutive rows i0 .. i0 + 3 of column j.
template <typename T, int Ph>
__device__ __forceinline__ void phase_epilogue(const SmallArgs& g, const SmallBucket& bk, const RoundBuffers& rb,
                                               int z, int i0, int j, const float v[4]) {
  if constexpr (Ph == 0) {
    GramEpi{bk.a32, g.first ? bk.scale : nullptr, bk.mp}(z, i0, j, v);
  } else if constexpr (Ph == 1) {
    PolyEpi{bk.a32, bk.phi, bk.plo, bk.plo == nullptr, g.sc, bk.mp}(z, i0, j, v);
  } else if constexpr (Ph == 2) {
    ApplyEpi<T>{reinterpret_cast<const T*>(rb.x_src), reinterpret_cast<T*>(rb.x_dst),
                reinterpret_cast<T*>(rb.xt_dst), g.first ? bk.scale : nullptr, g.sc, bk.mp, bk.np}(z, i0, j, v);
  } else {
    FinalEpi<T>{reinterpret_cast<const T*>(rb.x_src), g.first ? bk.scale : nullptr, g.sc, bk.mats, g.ptrs,
                bk.mp, bk.np, bk.m, bk.n}(z, i0, j, v);
  }
}

// ------------------------------------------------------------------ small products
// Buckets whose padded m is at most kSmallMaxMp (m <= 256).  One 32 x 32
// output tile per 256-thread workgroup; the contraction is split over the
// four waves: wave w takes k = 32 w .. 32 w + 31 of every 128-wide chunk,
// and the four partial sums are added in the fixed order ((w0 + w1) + w2) + w3.
// Chunks are double-buffered through registers into LDS; 16-byte chunk c of
// tile row r sits in slot c ^ (r mod 8), so the 16-byte fragment reads of 8
// consecutive rows hit distinct banks.
constexpr int kSmCK = 128;  // k elements per chunk (every padded dimension is a multiple of 128)

template <typename T, int Ph>
__global__ __launch_bounds__(256) void k_small(SmallArgs g) {
  constexpr int ES = (int)sizeof(T);
  constexpr int RB = kSmCK * ES;            // bytes of one tile row per chunk
  constexpr int CPR = RB / 16;              // 16-byte chunks per row
  constexpr int H = kSmallTile * CPR / 256; // 16-byte pieces per thread, operand and chunk
  constexpr int PH = grid_phase<Ph>();
  __shared__ __attribute__((aligned(16))) char lds[2][2][kSmallTile * RB];

  const int wg = blockIdx.x;
  const SmallBucket bk = find_bucket<PH>(g, wg);
  const RoundBuffers rbuf = round_buffers(bk, g.src);
  const int64_t tj_n = (PH == 2 ? bk.np : bk.mp) / kSmallTile, ti_n = bk.mp / kSmallTile;
  const int64_t local = wg - bk.t0[PH];
  const int z = (int)(local / (ti_n * tj_n));
  const int64_t t = local - (int64_t)z * ti_n * tj_n;
  const int ti = (int)(t / tj_n), tj = (int)(t - (t / tj_n) * tj_n);

  const Operands op = slice_operands<T, Ph>(bk, rbuf, z);
  const int64_t ld = op.ld;
  const char* A = op.a + (int64_t)ti * kSmallTile * ld * ES;
  const char* A2 = op.a2 ? op.a2 + (int64_t)ti * kSmallTile * ld * ES : nullptr;
  const char* B = op.b + (int64_t)tj * kSmallTile * ld * ES;
  const int nk = (int)(op.K / kSmCK);
  const int total = A2 ? 2 * nk : nk;  // with a bf16 hi/lo pair: the hi part's chunks, then the lo part's

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  u32x4_t ra[H], rb[H];
  auto gload = [&](int it) {
    const int kt = it % nk;
    const char* Ab = it >= nk ? A2 : A;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int p = tid + 256 * h, row = p / CPR, c = p % CPR;
      const int64_t off = (int64_t)row * ld * ES + (int64_t)kt * RB + c * 16;
      ra[h] = *reinterpret_cast<const MUON_GLOBAL u32x4_t*>(as_global(Ab + off));
      rb[h] = *reinterpret_cast<const MUON_GLOBAL u32x4_t*>(as_global(B + off));
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int p = tid + 256 * h, row = p / CPR, c = p % CPR;
      const int slot = row * RB + ((c ^ (row & 7)) << 4);
      *reinterpret_cast<u32x4_t*>(&lds[buf][0][slot]) = ra[h];
      *reinterpret_cast<u32x4_t*>(&lds[buf][1][slot]) = rb[h];
    }
  };
  // 16-byte fragment of row r at logical chunk c.
  auto frag = [&](const char* st, int r, int c) {
    return *reinterpret_cast<const u32x4_t*>(st + r * RB + ((c ^ (r & 7)) << 4));
  };

  f32x16_t acc = f32x16_t{};
  gload(0);
  sstore(0);
  __syncthreads();
  const int r = lane & 31, half = lane >> 5;
  for (int it = 0; it < total; ++it) {
    const int cur = it & 1;
    if (it + 1 < total) gload(it + 1);
    const char* As = lds[cur][0];
    const char* Bs = lds[cur][1];
    if constexpr (ES == 2) {
      // 32 k per wave: two 32x32x16 products; lane l holds k 8 (l/32) .. + 7 of each.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int c = 4 * wave + 2 * s2 + half;
        const u32x4_t av = frag(As, r, c), bv = frag(Bs, r, c);
        acc = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc);
      }
    } else {
      // 32 k per wave in 4 groups of 8: lane l reads 4 consecutive k (16 bytes)
      // at 8 s4 + 4 (l/32); product e adds k 8 s4 + e (lanes 0-31) and
      // 8 s4 + 4 + e (lanes 32-63).  A and B use the same k order.
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int c = 8 * wave + 2 * s4 + half;
        const f32x4_t av = __builtin_bit_cast(f32x4_t, frag(As, r, c));
        const f32x4_t bv = __builtin_bit_cast(f32x4_t, frag(Bs, r, c));
        acc = mfma_f32(av.x, bv.x, acc);
        acc = mfma_f32(av.y, bv.y, acc);
        acc = mfma_f32(av.z, bv.z, acc);
        acc = mfma_f32(av.w, bv.w, acc);
      }
    }
    if (it + 1 < total) sstore(cur ^ 1);
    __syncthreads();
  }

  // The four waves' partial tiles, added in a fixed order.  Accumulator
  // register q of lane l is row 8 (q/4) + 4 (l/32) + q mod 4, column l mod 32.
  float* red = reinterpret_cast<float*>(&lds[0][0][0]);  // [wave][32][33], over both buffers
  static_assert(4 * 32 * 33 * 4 <= (int)sizeof(lds), "the reduction buffer fits in the chunk buffers");
#pragma unroll
  for (int q = 0; q < 16; ++q) red[(wave * 32 + 8 * (q >> 2) + 4 * half + (q & 3)) * 33 + r] = acc[q];
  __syncthreads();
  const int col = tid & 31, i0 = 4 * (tid >> 5);
  float v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = (i0 + u) * 33 + col;
    v[u] = ((red[e] + red[32 * 33 + e]) + red[2 * 32 * 33 + e]) + red[3 * 32 * 33 + e];
  }
  phase_epilogue<T, Ph>(g, bk, rbuf, z, ti * kSmallTile + i0, tj * kSmallTile + col, v);
}

// ------------------------------------------------------------------ tiled products
// The other streamed buckets (padded m > 256 and not on the large tiles: the
// float32 mode, and bf16 slices the large tiles do not take).  BT x BT output
// tile per 256-thread workgroup (BT = 128, or 64 where the launch would have
// fewer 128-tiles than the chip has CUs); 4 waves in a 2 x 2 grid, each
// computing BT/2 x BT/2 with 32x32 matrix-core instructions.  k-slices of 64
// bytes per row are staged through LDS, double buffered.  Every output entry
// takes its k steps in the same order whatever BT is, so the tile size does
// not change a single bit of the result.
constexpr int kRowBytes = 64;       // bytes of k per operand row per stage
constexpr int kLdsRow = kRowBytes + 16;

template <typename T, int Ph, int BT>
__global__ __launch_bounds__(256) void k_mid(SmallArgs g) {
  constexpr int ES = (int)sizeof(T);
  constexpr int BK = kRowBytes / ES;
  constexpr int X = BT / 64;  // 32x32 blocks per wave along i and along j
  constexpr int H = BT / 64;  // 16-byte loads per thread, operand and slice
  constexpr int WT = BT / 2;  // rows (columns) per wave
  constexpr int PH = grid_phase<Ph>();
  __shared__ __attribute__((aligned(16))) char lds[2][2][BT * kLdsRow];

  const int wg = blockIdx.x;
  const SmallBucket bk = find_bucket<PH>(g, wg);
  const RoundBuffers rbuf = round_buffers(bk, g.src);
  const int64_t tj_n = (PH == 2 ? bk.np : bk.mp) / BT, ti_n = bk.mp / BT;
  const int64_t local = wg - bk.t0[PH];
  const int z = (int)(local / (ti_n * tj_n));
  const int64_t t = local - (int64_t)z * ti_n * tj_n;
  const int tm = (int)(t / tj_n), tn = (int)(t - (t / tj_n) * tj_n);

  const Operands op = slice_operands<T, Ph>(bk, rbuf, z);
  const int64_t ld = op.ld;
  const char* A = op.a + (int64_t)tm * BT * ld * ES;
  const char* A2 = op.a2 ? op.a2 + (int64_t)tm * BT * ld * ES : nullptr;
  const char* B = op.b + (int64_t)tn * BT * ld * ES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int row[H], c16[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int idx = tid + 256 * h;
    row[h] = idx >> 2;
    c16[h] = idx & 3;
  }
  u32x4_t ra[H], rb[H];
  const int nk = (int)(op.K / BK);
  const int total = A2 ? 2 * nk : nk;  // with a bf16 hi/lo pair: the hi part's slices, then the lo part's

  auto gload = [&](int it) {
    const int kt = it % nk;
    const char* Ab = it >= nk ? A2 : A;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t off = ((int64_t)row[h] * ld + (int64_t)kt * BK) * ES + c16[h] * 16;
      ra[h] = *reinterpret_cast<const MUON_GLOBAL u32x4_t*>(as_global(Ab + off));
      rb[h] = *reinterpret_cast<const MUON_GLOBAL u32x4_t*>(as_global(B + off));
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      *reinterpret_cast<u32x4_t*>(&lds[buf][0][row[h] * kLdsRow + c16[h] * 16]) = ra[h];
      *reinterpret_cast<u32x4_t*>(&lds[buf][1][row[h] * kLdsRow + c16[h] * 16]) = rb[h];
    }
  };

  f32x16_t acc[X][X];
#pragma unroll
  for (int x = 0; x < X; ++x)
#pragma unroll
    for (int y = 0; y < X; ++y) acc[x][y] = f32x16_t{};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int cur = it & 1;
    if (it + 1 < total) gload(it + 1);
    const char* As = lds[cur][0];
    const char* Bs = lds[cur][1];
    if constexpr (ES == 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t af[X], bf[X];
#pragma unroll
        for (int x = 0; x < X; ++x)
          af[x] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WT + x * 32 + (lane & 31)) * kLdsRow + s * 32 + (lane >> 5) * 16);
#pragma unroll
        for (int y = 0; y < X; ++y)
          bf[y] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WT + y * 32 + (lane & 31)) * kLdsRow + s * 32 + (lane >> 5) * 16);
#pragma unroll
        for (int x = 0; x < X; ++x)
#pragma unroll
          for (int y = 0; y < X; ++y) acc[x][y] = mfma_bf16(af[x], bf[y], acc[x][y]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float af[X], bf[X];
#pragma unroll
        for (int x = 0; x < X; ++x)
          af[x] = *reinterpret_cast<const float*>(As + (wm * WT + x * 32 + (lane & 31)) * kLdsRow + (s * 2 + (lane >> 5)) * 4);
#pragma unroll
        for (int y = 0; y < X; ++y)
          bf[y] = *reinterpret_cast<const float*>(Bs + (wn * WT + y * 32 + (lane & 31)) * kLdsRow + (s * 2 + (lane >> 5)) * 4);
#pragma unroll
        for (int x = 0; x < X; ++x)
#pragma unroll
          for (int y = 0; y < X; ++y) acc[x][y] = mfma_f32(af[x], bf[y], acc[x][y]);
      }
    }
    if (it + 1 < total) sstore(cur ^ 1);
    __syncthreads();
  }

  // Output layout of a 32x32 block: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, column l%32.
#pragma unroll
  for (int x = 0; x < X; ++x)
#pragma unroll
    for (int y = 0; y < X; ++y)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i0 = tm * BT + wm * WT + x * 32 + 8 * q + 4 * (lane >> 5);
        const int j = tn * BT + wn * WT + y * 32 + (lane & 31);
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = acc[x][y][4 * q + u];
        phase_epilogue<T, Ph>(g, bk, rbuf, z, i0, j, v);
      }
}

template <int BT>
void launch_mid_bt(int phase, bool final_round, bool f32_operands, const SmallArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (phase == 1) {
    hipLaunchKernelGGL((k_mid<float, 1, BT>), grid, block, 0, s, a);  // A is float32 in both modes
  } else if (phase == 0) {
    if (f32_operands) hipLaunchKernelGGL((k_mid<float, 0, BT>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_mid<uint16_t, 0, BT>), grid, block, 0, s, a);
  } else if (final_round) {
    if (f32_operands) hipLaunchKernelGGL((k_mid<float, 3, BT>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_mid<uint16_t, 3, BT>), grid, block, 0, s, a);
  } else {
    if (f32_operands) hipLaunchKernelGGL((k_mid<float, 2, BT>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_mid<uint16_t, 2, BT>), grid, block, 0, s, a);
  }
}

}  // namespace

hipError_t launch_prologue(DevScalars* dst, const DevScalars& v, hipStream_t s) {
  hipLaunchKernelGGL(k_prologue, dim3(1), dim3(64), 0, s, dst, v);
  return hipGetLastError();
}

hipError_t launch_momentum(const MomentumLaunch& a, hipStream_t s) {
  if (a.x_bytes == 2) hipLaunchKernelGGL(k_momentum<uint16_t>, dim3(a.km_tiles, a.count), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_momentum<float>, dim3(a.km_tiles, a.count), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm(const NormLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_norm, dim3(a.count), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_small(int phase, bool final_round, bool f32_operands, const SmallArgs& a, int64_t wgs,
                        hipStream_t s) {
  const dim3 grid((unsigned)wgs), block(256);
  if (phase == 1) {
    hipLaunchKernelGGL((k_small<float, 1>), grid, block, 0, s, a);  // A is float32 in both modes
  } else if (phase == 0) {
    if (f32_operands) hipLaunchKernelGGL((k_small<float, 0>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_small<uint16_t, 0>), grid, block, 0, s, a);
  } else if (final_round) {
    if (f32_operands) hipLaunchKernelGGL((k_small<float, 3>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_small<uint16_t, 3>), grid, block, 0, s, a);
  } else {
    if (f32_operands) hipLaunchKernelGGL((k_small<float, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_small<uint16_t, 2>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mid(int phase, bool final_round, bool f32_operands, const SmallArgs& a, int64_t wgs, int bt,
                      hipStream_t s) {
  const dim3 grid((unsigned)wgs);
  if (bt == 64) launch_mid_bt<64>(phase, final_round, f32_operands, a, grid, s);
  else launch_mid_bt<128>(phase, final_round, f32_operands, a, grid, s);
  return hipGetLastError();
}

hipError_t launch_update0(const Update0Launch& a, hipStream_t s) {
  int64_t blocks = (a.m * a.n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_update0, dim3((unsigned)blocks, a.count), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
