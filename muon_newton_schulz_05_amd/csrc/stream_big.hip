// stream_big.hip -- matrix products of the streamed path for large slices in
// bf16 mode (m > 512, dimensions padded to multiples of 256).
//
// Per Newton-Schulz round ("关于分布式Muon的想法整合及讨论" §2 and §6: the Gram
// matrix is recomputed each round; "MindSpore HyperParallel X 盘古,Muon优化器实现
// 6倍性能跃升", 三大性能挑战: the round is matrix products and additions):
//
//   gram   A = s2 X X^T, stored three ways: float32 A, the diagonal d = diag(A)
//          in float32, and E = A - diag(d) rounded to bf16 (the operand of
//          the next product);
//   poly   R = (a - 1) I + b A + c A^2 with
//            A^2 = E E + diag(d) A + A diag(d) - diag(d)^2,
//          where only E E runs on the matrix cores; R is rounded to bf16;
//   apply  X' = s (X + R X) = s (a X + (b A + c A^2) X); the X term enters the
//          accumulators exactly through an identity block on the matrix cores.
//
// Keeping the diagonal out of the bf16 operands and shifting the polynomial by
// the identity leaves bf16 rounding only on the small off-diagonal part of A
// and on R, whose spectrum is near zero once the iteration has converged.
// This is an arithmetic arrangement of the same iteration, not a different
// method.
//
// The kernel: 256 x 256 output tile per 256-thread workgroup, each of the
// four waves owning 128 x 128 (4 x 4 blocks of v_mfma_f32_32x32x16_bf16).
// Operand k-slices of 64 elements (128 bytes a row) go from HBM straight into
// LDS with gfx950's global_load_lds_dwordx4, two stages deep; lane l of a
// load lands at byte 16 l of its 1 KB destination, and each lane fetches the
// 16-byte chunk c of its row that belongs in slot c ^ ((row / 2) mod 8), so
// the 16-byte fragment reads of 16 consecutive rows hit distinct bank groups.
// Output tiles come from a table that the planner orders for cache reuse;
// workgroups are dealt to the 8 XCDs round robin, so workgroup b takes table
// entry (b mod 8) * T/8 + b/8 and every XCD walks a contiguous stretch.
// Symmetric products (X X^T, E E) list only tiles on or above the diagonal;
// an off-diagonal tile is also written to its mirror position.  The epilogue
// turns the accumulators around in LDS and writes whole rows of 16-byte
// pieces, in the tile's own orientation and, where needed, transposed.
#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

constexpr int kBK = 64;                       // bf16 elements of k per slice
constexpr int kStage = (kBigTile + kBigTile) * 128;  // bytes per stage
constexpr int kViewRow = 1, kViewCol = 2;

#define LDS_PTR __attribute__((address_space(3)))

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct BigCore {
  const char* a;          // row operand, matrix 0 (bf16, rows contiguous along k)
  const char* b;          // column operand, matrix 0
  int64_t lda, ldb;       // row strides in elements
  int64_t sa, sb;         // matrix strides in elements
  int64_t K;              // contraction length, multiple of kBK
  const uint32_t* tiles;  // tile table: tm | tn << 16, kNoTile for padding
  int t8;                 // table length (multiple of 8)
};

__device__ __forceinline__ void st_bf16x4(uint16_t* p, f32x4_t v) {
  *reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(p)) =
      u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
__device__ __forceinline__ f32x4_t ld_f32x4(const float* p) {
  return *reinterpret_cast<const MUON_GLOBAL f32x4_t*>(as_global(p));
}
__device__ __forceinline__ void st_f32x4(float* p, f32x4_t v) {
  *reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(p)) = v;
}

template <class Epi>
__global__ __launch_bounds__(256) void k_gemm_big(BigCore c, Epi epi) {
  constexpr int FM = 4, FN = 4;    // 32x32 blocks per wave along i and j
  constexpr int IA = 8, IB = 8;    // load instructions per wave and slice
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStage];

  int b = blockIdx.x;
  b = (b & 7) * (c.t8 >> 3) + (b >> 3);
  const uint32_t t = c.tiles[b];
  if (t == kNoTile) return;  // uniform over the workgroup, before any barrier
  const int tm = (int)(t & 0xFFFFu), tn = (int)(t >> 16);

  const int z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const char* A = c.a + ((int64_t)z * c.sa + (int64_t)tm * kBigTile * c.lda) * 2;
  const char* B = c.b + ((int64_t)z * c.sb + (int64_t)tn * kBigTile * c.ldb) * 2;
  const int nk = (int)(c.K / kBK);

  // Instruction u of wave w fills rows 8 (w + 4 u) .. + 7 of an operand tile.
  uint32_t oa[IA], ob[IB];
#pragma unroll
  for (int u = 0; u < IA; ++u) {
    const int row = 8 * (wave + 4 * u) + (lane >> 3);
    oa[u] = (uint32_t)(row * c.lda * 2 + (((lane & 7) ^ swz(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < IB; ++u) {
    const int row = 8 * (wave + 4 * u) + (lane >> 3);
    ob[u] = (uint32_t)(row * c.ldb * 2 + (((lane & 7) ^ swz(row)) << 4));
  }
  auto issue = [&](int kt, int stage) {
    char LDS_PTR* base = (char LDS_PTR*)(lds + stage * kStage);
#pragma unroll
    for (int u = 0; u < IA; ++u)
      __builtin_amdgcn_global_load_lds((const MUON_GLOBAL void*)(A + (int64_t)kt * 128 + oa[u]),
                                       (void LDS_PTR*)(base + (wave + 4 * u) * 1024), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < IB; ++u)
      __builtin_amdgcn_global_load_lds((const MUON_GLOBAL void*)(B + (int64_t)kt * 128 + ob[u]),
                                       (void LDS_PTR*)(base + kBigTile * 128 + (wave + 4 * u) * 1024), 16, 0, 0);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  const int ra = wm * 128 + (lane & 31), rb = kBigTile + wn * 128 + (lane & 31);
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, cur ^ 1);
      // This wave's loads of slice kt are the ones issued before the last IA + IB.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IA + IB) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // A bare barrier: the wait above already covers this wave's loads of
    // slice kt, and a fenced __syncthreads would also wait for slice kt + 1.
    __builtin_amdgcn_s_barrier();  // every wave's part of slice kt is in LDS
    const char* st = lds + cur * kStage;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int ck = 2 * s + (lane >> 5);
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = ra + 32 * i;
        af[i] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + ((ck ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = rb + 32 * j;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + ((ck ^ swz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
      if constexpr (Epi::kIdentity) {
        // acc += I B over the slices that run along the tile's own rows:
        // k-substep s of slice kt covers tile rows 64 (kt mod 4) + 16 s ..,
        // which lie in block blk of the waves with this wm.
        if ((kt >> 2) == tm) {
          const int blk = 2 * (kt & 3) + (s >> 1) - 4 * wm;
          if (blk >= 0 && blk < FM) {
            // Row operand lane l holds A[l mod 32][8 (l / 32) + e], e = 0..7.
            const int d = (lane & 31) - 16 * (s & 1) - 8 * (lane >> 5);
            bf16x8_t id;
#pragma unroll
            for (int e = 0; e < 8; ++e) id[e] = d == e ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
              if (i == blk) {
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(id, bfr[j], acc[i][j]);
              }
          }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // slice kt fully read before its stage is refilled
  }

  // ---- epilogue.  Accumulator layout of a 32x32 block: lane l, register r ->
  // row 8 (r / 4) + 4 (l / 32) + r mod 4, column l mod 32.  Half of the tile
  // (128 x 256 float32 = 128 KB) is staged at a time.
  const auto cx = epi.context(z);
  const int views = epi.views(cx, tm == tn);
  const float pre = epi.prescale(cx);
  float* stg = reinterpret_cast<float*>(lds);
  if (views & kViewRow) {
    // Row view: staged [i][j]; 16-byte slot s of row r sits at s ^ (8 ((r / 4) mod 2)).
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int r = i * 32 + 8 * q + 4 * (lane >> 5) + u;
                const int col = wn * 128 + j * 32 + (lane & 31);
                const int ps = (col >> 2) ^ (((r >> 2) & 1) << 3);
                stg[r * 256 + ps * 4 + (col & 3)] = pre * acc[i][j][4 * q + u];
              }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 32; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 6, s = idx & 63;
        const int ps = s ^ (((r >> 2) & 1) << 3);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + r * 256 + ps * 4);
        epi.store(cx, kViewRow, tm * kBigTile + h * 128 + r, tn * kBigTile + s * 4, v);
      }
      __syncthreads();
    }
  }
  if (views & kViewCol) {
    // Column view: staged [j][i] (four consecutive i per lane are one 16-byte
    // slot); slot s of row r sits at s ^ (r mod 16).
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      if (wn == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rc = j * 32 + (lane & 31);
              const int ci = wm * 128 + i * 32 + 8 * q + 4 * (lane >> 5);
              const int ps = (ci >> 2) ^ (rc & 15);
              f32x4_t v;
              v.x = pre * acc[i][j][4 * q + 0];
              v.y = pre * acc[i][j][4 * q + 1];
              v.z = pre * acc[i][j][4 * q + 2];
              v.w = pre * acc[i][j][4 * q + 3];
              *reinterpret_cast<f32x4_t*>(stg + rc * 256 + ps * 4) = v;
            }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 32; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 6, s = idx & 63;
        const int ps = s ^ (r & 15);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + r * 256 + ps * 4);
        epi.store(cx, kViewCol, tn * kBigTile + h * 128 + r, tm * kBigTile + s * 4, v);
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ epilogues
// store(cx, view, r, c, v): v holds entries (r, c .. c+3) of the output in the
// given view (kViewCol: of the transposed output); c is a multiple of 4.

// A = s2 X X^T: float32 A, float32 diagonal, bf16 A with a zero diagonal.
struct GramEpiBig {
  static constexpr bool kIdentity = false;
  float* a32;
  uint16_t* e16;
  float* dg;
  const float* scale;  // {s, s^2} per slice on the first round, else null
  int64_t mp;
  struct Ctx {
    float* a32;
    uint16_t* e16;
    float* dg;
    float pre;
  };
  __device__ Ctx context(int z) const {
    const int64_t o = (int64_t)z * mp * mp;
    return Ctx{a32 + o, e16 + o, dg + (int64_t)z * mp, scale ? scale[2 * z + 1] : 1.f};
  }
  __device__ float prescale(const Ctx& x) const { return x.pre; }
  __device__ int views(const Ctx&, bool diag) const { return diag ? kViewRow : kViewRow | kViewCol; }
  __device__ void store(const Ctx& x, int, int r, int c, f32x4_t v) const {
    const int64_t idx = (int64_t)r * mp + c;
    st_f32x4(x.a32 + idx, v);
    const int d = r - c;  // position of the diagonal in this piece, if any
    if (d >= 0 && d < 4) {
      const float dv = d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
      *reinterpret_cast<MUON_GLOBAL float*>(as_global(x.dg + r)) = dv;
      v.x = d == 0 ? 0.f : v.x;
      v.y = d == 1 ? 0.f : v.y;
      v.z = d == 2 ? 0.f : v.z;
      v.w = d == 3 ? 0.f : v.w;
    }
    st_bf16x4(x.e16 + idx, v);
  }
};

// R = (a - 1) I + b A + c (E E + diag(d) A + A diag(d) - diag(d)^2), in bf16.
struct PolyEpiBig {
  static constexpr bool kIdentity = false;
  const float* a32;
  const float* dg;
  uint16_t* r16;
  const DevScalars* sc;
  int64_t mp;
  struct Ctx {
    const float* a32;
    const float* dg;
    uint16_t* r16;
    float b, c, am1;
  };
  __device__ Ctx context(int z) const {
    const int64_t o = (int64_t)z * mp * mp;
    return Ctx{a32 + o, dg + (int64_t)z * mp, r16 + o, sc->b, sc->c, sc->a - 1.f};
  }
  __device__ float prescale(const Ctx&) const { return 1.f; }
  __device__ int views(const Ctx&, bool diag) const { return diag ? kViewRow : kViewRow | kViewCol; }
  __device__ void store(const Ctx& x, int, int r, int c, f32x4_t ee) const {
    const int64_t idx = (int64_t)r * mp + c;
    const f32x4_t a = ld_f32x4(x.a32 + idx);
    const float dr = *reinterpret_cast<const MUON_GLOBAL float*>(as_global(x.dg + r));
    const f32x4_t dc = ld_f32x4(x.dg + c);
    f32x4_t o;
#define MUON_POLY_ONE(comp, u)                                                      \
    {                                                                               \
      const bool on_diag = r == c + (u);                                            \
      const float a2 = ee.comp + (on_diag ? dr * dr : (dr + dc.comp) * a.comp);     \
      o.comp = x.b * a.comp + x.c * a2 + (on_diag ? x.am1 : 0.f);                   \
    }
    MUON_POLY_ONE(x, 0)
    MUON_POLY_ONE(y, 1)
    MUON_POLY_ONE(z, 2)
    MUON_POLY_ONE(w, 3)
#undef MUON_POLY_ONE
    st_bf16x4(x.r16 + idx, o);
  }
};

// X' = s (X + R X): written as X' [mp][np] and X'^T [np][mp].
struct ApplyEpiBig {
  static constexpr bool kIdentity = true;
  uint16_t* x_new;
  uint16_t* xt_new;
  const float* scale;
  int64_t mp, np;
  struct Ctx {
    uint16_t* x;
    uint16_t* xt;
    float pre;
  };
  __device__ Ctx context(int z) const {
    const int64_t o = (int64_t)z * mp * np;
    return Ctx{x_new + o, xt_new + o, scale ? scale[2 * z] : 1.f};
  }
  __device__ float prescale(const Ctx& x) const { return x.pre; }
  __device__ int views(const Ctx&, bool) const { return kViewRow | kViewCol; }
  __device__ void store(const Ctx& x, int view, int r, int c, f32x4_t v) const {
    if (view == kViewRow) st_bf16x4(x.x + (int64_t)r * np + c, v);
    else st_bf16x4(x.xt + (int64_t)r * mp + c, v);
  }
};

// Last round: W <- W - lr s (X + R X), through the slice's own layout (the row
// view for a slice stored [m, n], the column view for one stored [n, m]).
struct FinalEpiBig {
  static constexpr bool kIdentity = true;
  const DevMat* mats;
  const PtrEntry* ptrs;
  const float* scale;
  const DevScalars* sc;
  int64_t m, n;
  int vec;  // rows of W are whole 16-byte groups (m and n multiples of 4)
  struct Ctx {
    char* w;
    int64_t rows, len;  // stored rows and row length of this slice
    int pdtype;
    float pre;
    int view;
  };
  __device__ Ctx context(int z) const {
    const DevMat d = mats[z];
    const PtrEntry pe = ptrs[d.param];
    const int esz = d.pdtype == 1 ? 2 : 4;
    Ctx x;
    x.w = static_cast<char*>(pe.w) + d.slice_off * esz;
    x.rows = d.transposed ? n : m;
    x.len = d.transposed ? m : n;
    x.pdtype = d.pdtype;
    x.pre = sc->lr * (scale ? scale[2 * z] : 1.f);
    x.view = d.transposed ? kViewCol : kViewRow;
    return x;
  }
  __device__ float prescale(const Ctx&) const { return 1.f; }
  __device__ int views(const Ctx& x, bool) const { return x.view; }
  __device__ void store(const Ctx& x, int, int r, int c, f32x4_t v) const {
    if (r >= x.rows || c >= x.len) return;
    const int64_t idx = (int64_t)r * x.len + c;
    if (vec && c + 3 < x.len) {
      if (x.pdtype == 1) {  // bfloat16 W
        MUON_GLOBAL u32x2_t* p = reinterpret_cast<MUON_GLOBAL u32x2_t*>(as_global(x.w) + 2 * idx);
        const u32x2_t w = *p;
        *p = u32x2_t{pack_bf16x2(bf16_lo(w.x) - x.pre * v.x, bf16_hi(w.x) - x.pre * v.y),
                     pack_bf16x2(bf16_lo(w.y) - x.pre * v.z, bf16_hi(w.y) - x.pre * v.w)};
      } else {
        MUON_GLOBAL f32x4_t* p = reinterpret_cast<MUON_GLOBAL f32x4_t*>(as_global(x.w) + 4 * idx);
        const f32x4_t w = *p;
        *p = f32x4_t{w.x - x.pre * v.x, w.y - x.pre * v.y, w.z - x.pre * v.z, w.w - x.pre * v.w};
      }
      return;
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c + u < x.len) {
        const float w = load_as_f32(x.w, idx + u, x.pdtype);
        store_from_f32(x.w, idx + u, x.pdtype, w - x.pre * vv[u]);
      }
    }
  }
};

template <class Epi>
hipError_t run_big(const BigCore& c, const Epi& e, int count, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_big<Epi>, dim3(c.t8, 1, count), dim3(256), 0, s, c, e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram_big(const GramBigLaunch& a, hipStream_t s) {
  BigCore c{};
  c.a = c.b = static_cast<const char*>(a.x);
  c.lda = c.ldb = a.np;
  c.sa = c.sb = a.mp * a.np;
  c.K = a.np;
  c.tiles = a.tiles;
  c.t8 = a.t8;
  return run_big(c, GramEpiBig{a.a32, a.e16, a.dg, a.scale, a.mp}, a.count, s);
}

hipError_t launch_poly_big(const PolyBigLaunch& a, hipStream_t s) {
  BigCore c{};
  c.a = c.b = reinterpret_cast<const char*>(a.e16);
  c.lda = c.ldb = a.mp;
  c.sa = c.sb = a.mp * a.mp;
  c.K = a.mp;
  c.tiles = a.tiles;
  c.t8 = a.t8;
  return run_big(c, PolyEpiBig{a.a32, a.dg, a.r16, a.sc, a.mp}, a.count, s);
}

hipError_t launch_apply_big(const ApplyBigLaunch& a, hipStream_t s) {
  BigCore c{};
  c.a = reinterpret_cast<const char*>(a.r16);
  c.b = static_cast<const char*>(a.xt_old);
  c.lda = a.mp;
  c.ldb = a.mp;
  c.sa = a.mp * a.mp;
  c.sb = a.np * a.mp;
  c.K = a.mp;
  c.tiles = a.tiles;
  c.t8 = a.t8;
  if (a.final_round) {
    const int vec = (a.m % 4 == 0) && (a.n % 4 == 0);
    return run_big(c, FinalEpiBig{a.mats, a.ptrs, a.scale, a.sc, a.m, a.n, vec}, a.count, s);
  }
  return run_big(c, ApplyEpiBig{static_cast<uint16_t*>(a.x_new), static_cast<uint16_t*>(a.xt_new),
                                a.scale, a.mp, a.np},
                 a.count, s);
}

}  // namespace muon
