// gemm_bf16.hip -- bf16 MFMA GEMM for gfx950 (CDNA4) with fused epilogues.
//
// Every matrix product of the shard (MLP, SwiGLU, attention projections, LM
// head; forward and backward) runs through this one kernel template.  The
// products are the column- and row-parallel GEMMs of the pages (book "7.3 模型
// 并行与张量并行" §7.3.2-§7.3.4, lecture 16 notes §5.2-§5.5); the element-wise
// activation, its derivative and the SwiGLU gating run in the epilogue, so the
// [s, f/t] intermediates are written once and read once.
//
// Design (MI355X first):
//  * 256 threads = 4 wave64s in a 2x2 grid; a workgroup computes a BMxBN tile,
//    each wave a (BM/2)x(BN/2) sub-tile of 32x32 v_mfma_f32_32x32x16_bf16 blocks
//    accumulated in fp32.
//  * K advances 64 at a time.  Tiles are staged global -> registers -> LDS with
//    two LDS buffers: the next tile's global loads are in flight while the
//    MFMAs consume the current buffer, one barrier per K step.
//  * LDS holds every operand tile as [rows][64 k] with 16-byte chunks XOR-
//    swizzled by (row ^ row>>3) & 7, so fragment reads (32 rows, one chunk)
//    and the staging writes are free of bank conflicts.
//  * Operands stored with k contiguous are copied chunk by chunk; operands
//    stored with m/n contiguous (weights [in,out] in X.W, X^T in X^T.dZ) are
//    loaded as 8x8 blocks and transposed in registers on the way to LDS.
//  * Workgroup ids are remapped so that consecutive tiles land on the same XCD
//    (each XCD has its own L2), then grouped along M for panel reuse.
#include <type_traits>

#include "gemm_desc.h"
#include "launch.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int NTHREADS = 256;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

__device__ __forceinline__ uint32_t elem16(const u32x4 &v, int i) {
  uint32_t w = v[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// Operand tile with k contiguous in memory: R rows x 64 k, R/32 16-byte
// chunks per thread.  Thread t takes chunk (t & 7) of rows (t >> 3) + 32 i.
template <int R, bool VEC>
struct LoadKC {
  u32x4 v[R / 32];
  __device__ __forceinline__ void load(const uint16_t *p, int64_t ld, int row0, int rows,
                                       int k0, int klen, int tid) {
    const int c = tid & 7;
    const int k = k0 + c * 8;
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
      const int row = row0 + (tid >> 3) + 32 * i;
      if (VEC) {
        v[i] = (row < rows && k < klen) ? *(const u32x4 *)(p + (int64_t)row * ld + k) : zero4();
      } else {
        u32x4 t = zero4();
        if (row < rows) {
          const uint16_t *q = p + (int64_t)row * ld;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t x = (k + e < klen) ? q[k + e] : 0u;
            t[e >> 1] |= (e & 1) ? (x << 16) : x;
          }
        }
        v[i] = t;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
      const int r = (tid >> 3) + 32 * i;
      lds[r * 8 + (c ^ swz(r))] = v[i];
    }
  }
};

// Operand tile with the row index (m or n) contiguous in memory: the thread
// owning 8x8 block (kb, rb) loads 8 k-rows of 8 consecutive elements and
// transposes them so that LDS row rb*8+i holds 8 consecutive k values.
// Rows >= `half` come from a second matrix p1 (the dual gate/up operand).
template <int R, bool VEC>
struct LoadRC {
  static constexpr int RB = R / 8;  // row blocks
  u32x4 v[8];
  __device__ __forceinline__ void load(const uint16_t *p0, const uint16_t *p1, int half,
                                       int64_t ld, int row0, int rows, int k0, int klen,
                                       int tid) {
    const int rb = tid % RB, kb = tid / RB;
    if (kb >= 8) return;
    int r = rb * 8;
    const uint16_t *p = p0;
    if (r >= half) { p = p1; r -= half; }
    const int col = row0 + r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + kb * 8 + e;
      if (VEC) {
        v[e] = (k < klen && col < rows) ? *(const u32x4 *)(p + (int64_t)k * ld + col) : zero4();
      } else {
        u32x4 t = zero4();
        if (k < klen) {
          const uint16_t *q = p + (int64_t)k * ld;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            uint32_t x = (col + i < rows) ? q[col + i] : 0u;
            t[i >> 1] |= (i & 1) ? (x << 16) : x;
          }
        }
        v[e] = t;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
    const int rb = tid % RB, kb = tid / RB;
    if (kb >= 8) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = elem16(v[2 * q], i) | (elem16(v[2 * q + 1], i) << 16);
      const int r = rb * 8 + i;
      lds[r * 8 + (kb ^ swz(r))] = o;
    }
  }
};

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ u32x4 pack8(const float *v) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (uint32_t)tp_f2bf(v[2 * q]) | ((uint32_t)tp_f2bf(v[2 * q + 1]) << 16);
  return o;
}

__device__ __forceinline__ void unpack8(const u32x4 &w, float *v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}

// Apply the epilogue to 8 consecutive columns gn..gn+7 of row gm (gm < M and
// gn < nlen checked by the caller).  In VEC mode a full run of 8 uses 16-byte
// accesses; a ragged tail (or the scalar build) goes element by element.
template <int EPI, bool OUT_F32, bool VEC>
__device__ __forceinline__ void epi8(const GemmDesc &d, int gm, int gn, int nlen, int sc, int split,
                                     const float *x, const float *u) {
  const int cnt = min(8, nlen - gn);
  const bool full = VEC && cnt == 8;
  if constexpr (EPI == EPI_PARTIAL) {
    const int col = d.kseg ? gn : d.seg_col0[sc] + gn;
    float *o = d.ws + ((int64_t)split * d.M + gm) * d.N + col;
    if (full) {
      *(float4 *)o = make_float4(x[0], x[1], x[2], x[3]);
      *(float4 *)(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else {
      for (int q = 0; q < cnt; ++q) o[q] = x[q];
    }
  } else if constexpr (EPI == EPI_STORE && OUT_F32) {
    float *o = (float *)d.C[sc] + (int64_t)gm * d.ldc[sc] + gn;
    if (full) {
      *(float4 *)o = make_float4(x[0], x[1], x[2], x[3]);
      *(float4 *)(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else {
      for (int q = 0; q < cnt; ++q) o[q] = x[q];
    }
  } else {
    // every other epilogue stores bf16 to C (and possibly ao0 / ao1)
    float y[8], y2[8];
    float a0[8], a1[8];
    const bool has_ai = EPI == EPI_ACT_BWD || EPI == EPI_SWIGLU_BWD;
    if constexpr (has_ai) {
      const int64_t o = (int64_t)gm * d.ldai + gn;
      if (full) {
        unpack8(*(const u32x4 *)((const uint16_t *)d.ai0 + o), a0);
        if constexpr (EPI == EPI_SWIGLU_BWD) unpack8(*(const u32x4 *)((const uint16_t *)d.ai1 + o), a1);
      } else {
        for (int q = 0; q < 8; ++q) {
          a0[q] = q < cnt ? tp_bf2f(((const uint16_t *)d.ai0)[o + q]) : 0.f;
          if constexpr (EPI == EPI_SWIGLU_BWD) a1[q] = q < cnt ? tp_bf2f(((const uint16_t *)d.ai1)[o + q]) : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if constexpr (EPI == EPI_STORE) {
        y[q] = x[q];
      } else if constexpr (EPI == EPI_ACT_FWD) {
        y[q] = tp_act_fwd(d.act, x[q]);
      } else if constexpr (EPI == EPI_ACT_BWD) {
        y[q] = x[q] * tp_act_grad(d.act, a0[q]);
      } else if constexpr (EPI == EPI_SWIGLU_FWD) {
        y[q] = x[q] * tp_sigmoid(x[q]) * u[q];
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const float g = a0[q], sg = tp_sigmoid(g);
        y[q] = x[q] * a1[q] * (sg * (1.f + g * (1.f - sg)));
        y2[q] = x[q] * g * sg;
      }
    }
    uint16_t *C = (uint16_t *)d.C[sc] + (int64_t)gm * d.ldc[sc] + gn;
    uint16_t *O0 = (uint16_t *)d.ao0 + (int64_t)gm * d.ldao + gn;
    uint16_t *O1 = (uint16_t *)d.ao1 + (int64_t)gm * d.ldao + gn;
    const bool w_o0 = (EPI == EPI_ACT_FWD && d.ao0) || EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD;
    if (full) {
      *(u32x4 *)C = pack8(y);
      if constexpr (EPI == EPI_ACT_FWD || EPI == EPI_SWIGLU_FWD) {
        if (w_o0) *(u32x4 *)O0 = pack8(x);
      }
      if constexpr (EPI == EPI_SWIGLU_FWD) *(u32x4 *)O1 = pack8(u);
      if constexpr (EPI == EPI_SWIGLU_BWD) *(u32x4 *)O0 = pack8(y2);
    } else {
      for (int q = 0; q < cnt; ++q) {
        C[q] = tp_f2bf(y[q]);
        if constexpr (EPI == EPI_ACT_FWD || EPI == EPI_SWIGLU_FWD) {
          if (w_o0) O0[q] = tp_f2bf(x[q]);
        }
        if constexpr (EPI == EPI_SWIGLU_FWD) O1[q] = tp_f2bf(u[q]);
        if constexpr (EPI == EPI_SWIGLU_BWD) O0[q] = tp_f2bf(y2[q]);
      }
    }
  }
}

template <int BM, int BN>
struct Smem {
  u32x4 a[2][BM * 8];
  u32x4 b[2][BN * 8];
};

__device__ __forceinline__ void tile_coords(const GemmDesc &d, int &tm, int &tn, int &split) {
  // XCD-aware remap: hardware deals workgroup ids round-robin over 8 XCDs;
  // give each XCD a contiguous range of logical tiles.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7, idx = bid >> 3;
  const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int tiles = d.tiles_m * d.tiles_n;
  split = lid / tiles;
  const int t = lid - split * tiles;
  const int in_group = d.group_m * d.tiles_n;
  const int g = t / in_group;
  const int first = g * d.group_m;
  const int gsz = min(d.tiles_m - first, d.group_m);
  const int w = t - g * in_group;
  tm = first + w % gsz;
  tn = w / gsz;
}

template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool VEC>
__global__ void __launch_bounds__(NTHREADS) gemm_bf16_kernel(GemmDesc d) {
  __shared__ Smem<BM, BN> sm;
  constexpr int WTM = BM / 2, WTN = BN / 2, FM = WTM / 32, FN = WTN / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  int tm, tn, split;
  tile_coords(d, tm, tn, split);

  int sn = 0;  // N-segment of this tile
  if (!d.kseg)
    while (sn + 1 < d.nseg && tn >= d.seg_tile0[sn + 1]) ++sn;
  const int ncols = d.dual ? BN / 2 : BN;
  const int n0 = d.kseg ? tn * BN : (tn - d.seg_tile0[sn]) * ncols;
  const int nlen = d.kseg ? d.N : d.seg_len[sn];
  const int m0 = tm * BM;

  const int kt_total = d.kseg ? d.seg_tile0[d.nseg] : (d.K + BK - 1) / BK;
  const int kt_begin = split * d.kt_per_split;
  const int kt_end = min(kt_total, kt_begin + d.kt_per_split);

  typename std::conditional<A_KC, LoadKC<BM, VEC>, LoadRC<BM, VEC>>::type la;
  typename std::conditional<B_KC, LoadKC<BN, VEC>, LoadRC<BN, VEC>>::type lb;

  auto load_tile = [&](int kt) {
    int ks = 0;
    if (d.kseg)
      while (ks + 1 < d.nseg && kt >= d.seg_tile0[ks + 1]) ++ks;
    const int k0 = d.kseg ? (kt - d.seg_tile0[ks]) * BK : kt * BK;
    const int klen = d.kseg ? d.seg_len[ks] : d.K;
    const int ia = d.kseg ? ks : 0;
    const int ib = d.kseg ? ks : sn;
    const uint16_t *Ap = (const uint16_t *)d.A[ia];
    const uint16_t *Bp = (const uint16_t *)d.B[ib];
    if constexpr (A_KC) la.load(Ap, d.lda[ia], m0, d.M, k0, klen, tid);
    else la.load(Ap, Ap, BM, d.lda[ia], m0, d.M, k0, klen, tid);
    if constexpr (B_KC) lb.load(Bp, d.ldb[ib], n0, nlen, k0, klen, tid);
    else lb.load(Bp, d.dual ? (const uint16_t *)d.B[1] : Bp, d.dual ? BN / 2 : BN, d.ldb[ib],
                 n0, nlen, k0, klen, tid);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // LDS row of the wave's fn-th 32-wide B fragment
  auto brow = [&](int fn) -> int {
    if (d.dual) {
      return (fn < FN / 2) ? wn * (BN / 4) + fn * 32 : BN / 2 + wn * (BN / 4) + (fn - FN / 2) * 32;
    }
    return wn * WTN + fn * 32;
  };

  if (kt_begin < kt_end) {
    load_tile(kt_begin);
    la.store(sm.a[0], tid);
    lb.store(sm.b[0], tid);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) load_tile(kt + 1);
    const u32x4 *As = sm.a[buf];
    const u32x4 *Bs = sm.b[buf];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WTM + fm * 32 + (lane & 31);
        af[fm] = __builtin_bit_cast(bf16x8, As[r * 8 + (kc ^ swz(r))]);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = brow(fn) + (lane & 31);
        bfr[fn] = __builtin_bit_cast(bf16x8, Bs[r * 8 + (kc ^ swz(r))]);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    }
    if (more) {
      la.store(sm.a[buf ^ 1], tid);
      lb.store(sm.b[buf ^ 1], tid);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Each wave stages one 32-row strip of its accumulators at a time through
  // LDS (fp32, rows padded by 8 floats so the MFMA-layout writes of the two
  // half-waves fall on different banks), then reads rows back as runs of 8
  // consecutive columns: the activation math runs once per element and every
  // global access is 16 bytes wide.
  // 32x32 accumulator layout: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32 of the block.
  constexpr int EPS = WTN + 8;                      // strip row stride (floats)
  constexpr bool DUALE = EPI == EPI_SWIGLU_FWD;
  constexpr int OUTW = DUALE ? WTN / 2 : WTN;       // output columns per strip row
  constexpr int LPR = OUTW / 8;                     // lanes per strip row
  constexpr int RPI = 64 / LPR;                     // strip rows per pass
  float *ep = (float *)&sm + wid * 32 * EPS;
  const int ci = lane & 31;
  const int rsub = 4 * (lane >> 5);
  const int col_base = n0 + (DUALE ? wn * (BN / 4) : wn * WTN);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    __syncthreads();
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ep[(8 * (e >> 2) + rsub + (e & 3)) * EPS + fn * 32 + ci] = acc[fm][fn][e];
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = it * RPI + lane / LPR;
      const int c = (lane % LPR) * 8;
      const float *src = ep + r * EPS + c;
      float x[8], u[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = src[q];
      if constexpr (DUALE) {
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = src[OUTW + q];
      }
      const int gm = m0 + wm * WTM + fm * 32 + r;
      const int gn = col_base + c;
      if (gm < d.M && gn < nlen)
        epi8<EPI, OUT_F32, VEC>(d, gm, gn, nlen, d.kseg ? 0 : sn, split, x, u);
    }
  }
}

// Sum the split-K partials in split order (deterministic) and store.
template <bool OUT_F32>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmDesc d) {
  const int64_t total = (int64_t)d.M * d.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int gm = (int)(i / d.N), gc = (int)(i - (int64_t)gm * d.N);
    float s = 0.f;
    for (int k = 0; k < d.splits; ++k) s += d.ws[((int64_t)k * d.M + gm) * d.N + gc];
    int sg = 0;
    if (!d.kseg)
      while (sg + 1 < d.nseg && gc >= d.seg_col0[sg + 1]) ++sg;
    const int cc = d.kseg ? gc : gc - d.seg_col0[sg];
    const int si = d.kseg ? 0 : sg;
    if (OUT_F32) ((float *)d.C[si])[(int64_t)gm * d.ldc[si] + cc] = s;
    else ((uint16_t *)d.C[si])[(int64_t)gm * d.ldc[si] + cc] = tp_f2bf(s);
  }
}

template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool VEC>
hipError_t launch_tiles(const GemmDesc &d, hipStream_t st) {
  const int nblk = d.tiles_m * d.tiles_n * d.splits;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_KC, B_KC, EPI, OUT_F32, VEC>), dim3(nblk),
                     dim3(NTHREADS), 0, st, d);
  return hipGetLastError();
}

template <bool A_KC, bool B_KC, int EPI, bool OUT_F32>
hipError_t launch_shape(const GemmDesc &d, int bm, int bn, hipStream_t st, bool vec) {
  // the scalar-load build exists only for 128x128 tiles (odd sizes are small)
  if (!vec) return launch_tiles<128, 128, A_KC, B_KC, EPI, OUT_F32, false>(d, st);
  if (bm == 256 && bn == 256) return launch_tiles<256, 256, A_KC, B_KC, EPI, OUT_F32, true>(d, st);
  if (bm == 256 && bn == 128) return launch_tiles<256, 128, A_KC, B_KC, EPI, OUT_F32, true>(d, st);
  if (bm == 128 && bn == 256) return launch_tiles<128, 256, A_KC, B_KC, EPI, OUT_F32, true>(d, st);
  return launch_tiles<128, 128, A_KC, B_KC, EPI, OUT_F32, true>(d, st);
}

}  // namespace

// Launch one planned bf16 product.  `layout`: GEMM_NN (A k-contig, B n-contig),
// GEMM_NT (both k-contig), GEMM_TN (A m-contig, B n-contig).
hipError_t tp_launch_gemm_bf16(const GemmDesc &d, int layout, int epi, bool out_f32, int bm, int bn,
                               bool vec, hipStream_t st) {
  hipError_t e = hipSuccess;
  switch (layout) {
  case GEMM_NN:
    switch (epi) {
    case EPI_STORE:
      e = out_f32 ? launch_shape<true, false, EPI_STORE, true>(d, bm, bn, st, vec)
                  : launch_shape<true, false, EPI_STORE, false>(d, bm, bn, st, vec);
      break;
    case EPI_ACT_FWD: e = launch_shape<true, false, EPI_ACT_FWD, false>(d, bm, bn, st, vec); break;
    case EPI_SWIGLU_FWD: e = launch_shape<true, false, EPI_SWIGLU_FWD, false>(d, bm, bn, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<true, false, EPI_PARTIAL, true>(d, bm, bn, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  case GEMM_NT:
    switch (epi) {
    case EPI_STORE: e = launch_shape<true, true, EPI_STORE, false>(d, bm, bn, st, vec); break;
    case EPI_ACT_BWD: e = launch_shape<true, true, EPI_ACT_BWD, false>(d, bm, bn, st, vec); break;
    case EPI_SWIGLU_BWD: e = launch_shape<true, true, EPI_SWIGLU_BWD, false>(d, bm, bn, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<true, true, EPI_PARTIAL, true>(d, bm, bn, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  case GEMM_TN:
    switch (epi) {
    case EPI_STORE: e = launch_shape<false, false, EPI_STORE, false>(d, bm, bn, st, vec); break;
    case EPI_PARTIAL: e = launch_shape<false, false, EPI_PARTIAL, true>(d, bm, bn, st, vec); break;
    default: return hipErrorInvalidValue;
    }
    break;
  default: return hipErrorInvalidValue;
  }
  return e;
}

hipError_t tp_launch_splitk_reduce(const GemmDesc &d, bool out_f32, hipStream_t st) {
  const int64_t total = (int64_t)d.M * d.N;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (out_f32) hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, d);
  else hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, d);
  return hipGetLastError();
}
