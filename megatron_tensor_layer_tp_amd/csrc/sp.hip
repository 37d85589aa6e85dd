// sp.hip -- the sequence-parallel region of a layer on one shard's positions:
// residual add with dropout, then LayerNorm, and the backward of both
// ("7.3 模型并行与张量并行" §7.3.6: LayerNorm and dropout act on each position
// independently, so between a sublayer's reduce-scatter and the next sublayer's
// all-gather each card keeps only its s/t positions).
//
//   forward   u = x + y * mask / (1 - p),  z = (u - mean) * rstd * gamma + beta
//   backward  du = dun + rstd * (g - mean(g) - xh * mean(g * xh)),  g = dz * gamma,
//             dx = du,  dy = du * mask / (1 - p),
//             dgamma = sum_rows dz * xh,  dbeta = sum_rows dz
//
// HBM-streaming kernels.  One 256-thread workgroup per row: every element of
// the row is loaded once into registers (16-byte loads of 8 bf16 when h is a
// multiple of 8), the row statistics are exact two-pass sums over those
// registers (wave shuffles, then LDS across the 4 waves), and every output is
// written once.  The backward's dgamma / dbeta are column sums over the rows.
// For rows of up to 8192 columns in 16-byte vectors the row kernel keeps them:
// each of its 256 workgroups sums its own rows (in increasing order) in
// registers and writes one partial; otherwise a second kernel sums chunks of 16
// rows per column into partials.  Either way a last kernel reduces the partials
// in a fixed order (deterministic); when h is a multiple of 64 the row kernel
// lays its partials out by 64-column block, so that each workgroup of that
// reduction reads one contiguous run.
#include "launch.h"

namespace {

constexpr int SP_THREADS = 256;
constexpr int SP_VPT = 4;  // 8-element vectors per thread and pass (a pass covers 8192 columns)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void unpack8(const u32x4 &w, float *v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const float *v) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2_t p = {v[2 * q], v[2 * q + 1]};
    o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
  }
  return o;
}

// sum over the workgroup (every thread gets the total); `red` holds 4 floats
__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// column c of vector slot i of this thread: element 8 * (tid + 256 i) + q
template <bool VEC>
__device__ __forceinline__ int col_of(int i, int q) {
  return VEC ? 8 * ((int)threadIdx.x + SP_THREADS * i) + q : (int)threadIdx.x + SP_THREADS * (8 * i + q);
}

// load 8 elements (VEC: one 16-byte vector; else strided scalars, 0 past the row end)
template <bool VEC>
__device__ __forceinline__ void load8(const uint16_t *row, int i, int h, float *v) {
  if constexpr (VEC) {
    const int c = col_of<true>(i, 0);
    if (c < h) unpack8(*(const u32x4 *)(row + c), v);
    else
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.f;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = col_of<false>(i, q);
      v[q] = c < h ? bf2f(row[c]) : 0.f;
    }
  }
}
template <bool VEC>
__device__ __forceinline__ void mask8(const uint8_t *row, int i, int h, float *v) {
  if constexpr (VEC) {
    const int c = col_of<true>(i, 0);
    if (c < h) {
      const uint2 m = *(const uint2 *)(row + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (float)((m.x >> (8 * q)) & 0xffu);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 + q] = (float)((m.y >> (8 * q)) & 0xffu);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = col_of<false>(i, q);
      v[q] = c < h ? (float)row[c] : 0.f;
    }
  }
}
template <bool VEC>
__device__ __forceinline__ void store8(uint16_t *row, int i, int h, const float *v) {
  if constexpr (VEC) {
    const int c = col_of<true>(i, 0);
    if (c < h) *(u32x4 *)(row + c) = pack8(v);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = col_of<false>(i, q);
      if (c < h) row[c] = f2bf(v[q]);
    }
  }
}

// the same 8 elements kept packed until used (4 registers instead of 8): bf16 bits and mask bytes
template <bool VEC>
__device__ __forceinline__ u32x4 raw8(const uint16_t *row, int i, int h) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if constexpr (VEC) {
    const int c = col_of<true>(i, 0);
    if (c < h) w = *(const u32x4 *)(row + c);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = col_of<false>(i, q);
      if (c < h) w[q >> 1] |= (uint32_t)row[c] << (16 * (q & 1));
    }
  }
  return w;
}
template <bool VEC>
__device__ __forceinline__ uint2 rawmask8(const uint8_t *row, int i, int h) {
  uint2 m = make_uint2(0u, 0u);
  if constexpr (VEC) {
    const int c = col_of<true>(i, 0);
    if (c < h) m = *(const uint2 *)(row + c);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = col_of<false>(i, q);
      if (c < h) {
        if (q < 4) m.x |= (uint32_t)row[c] << (8 * q);
        else m.y |= (uint32_t)row[c] << (8 * (q - 4));
      }
    }
  }
  return m;
}
__device__ __forceinline__ float mask_at(const uint2 &m, int q) {
  return (float)(((q < 4 ? m.x : m.y) >> (8 * (q & 3))) & 0xffu);
}

// the same 16-byte row loads, non-temporal: the forward reads each row once
// (22 -> 18.4 us on the c4 slice in the step; the backward measured 3% slower
// with them and keeps plain loads)
__device__ __forceinline__ u32x4 raw8_nt(const uint16_t *row, int c, int h) {
  return c < h ? __builtin_nontemporal_load((const u32x4 *)(row + c)) : u32x4{0u, 0u, 0u, 0u};
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 rawmask8_nt(const uint8_t *row, int c, int h) {
  if (c >= h) return make_uint2(0u, 0u);
  const u32x2 m = __builtin_nontemporal_load((const u32x2 *)(row + c));
  return make_uint2(m[0], m[1]);
}

struct SpArgs {
  int64_t n, h;
  float keep, eps;  // 1 / (1 - p), LayerNorm epsilon
  const uint16_t *y, *x, *gamma, *beta, *dz, *dun, *u;
  const uint8_t *mask;
  uint16_t *uo, *z, *dx, *dy, *dgamma, *dbeta;
  float *mean, *rstd, *part;  // part: [row chunks][2][h] partial column sums
};

// rows of up to SP_VPT * 8 * 256 = 8192 columns in registers (NP passes for longer rows)
template <bool VEC, int NP>
__global__ void __launch_bounds__(SP_THREADS) sp_ln_fwd_kernel(SpArgs a) {
  __shared__ float red[4];
  const int h = (int)a.h;
  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    const uint16_t *yr = a.y + r * a.h, *xr = a.x + r * a.h;
    const uint8_t *mr = a.mask + r * a.h;
    float u[NP * SP_VPT][8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NP * SP_VPT; ++i) {
      float yv[8], xv[8], mv[8];
      load8<VEC>(yr, i, h, yv);
      load8<VEC>(xr, i, h, xv);
      mask8<VEC>(mr, i, h, mv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        u[i][q] = fmaf(yv[q] * mv[q], a.keep, xv[q]);
        s += u[i][q];
      }
    }
    const float mean = block_sum(s, red) / (float)h;
    float v2 = 0.f;
#pragma unroll
    for (int i = 0; i < NP * SP_VPT; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = col_of<VEC>(i, q) < h;
        const float d = u[i][q] - mean;
        v2 += in ? d * d : 0.f;
      }
    const float var = block_sum(v2, red) / (float)h;
    const float rstd = 1.f / sqrtf(var + a.eps);
    uint16_t *ur = a.uo + r * a.h, *zr = a.z + r * a.h;
#pragma unroll
    for (int i = 0; i < NP * SP_VPT; ++i) {
      // gamma and beta are shared by every row: L2 hits
      float zv[8], gv[8], bv[8];
      load8<VEC>(a.gamma, i, h, gv);
      load8<VEC>(a.beta, i, h, bv);
#pragma unroll
      for (int q = 0; q < 8; ++q) zv[q] = fmaf((u[i][q] - mean) * rstd, gv[q], bv[q]);
      store8<VEC>(ur, i, h, u[i]);
      store8<VEC>(zr, i, h, zv);
    }
    if (threadIdx.x == 0) {
      a.mean[r] = mean;
      a.rstd[r] = rstd;
    }
  }
}

// Rows of at most 8192 columns (h % 8 == 0), several rows per workgroup: the
// next row's y, x and mask are loaded before this row's stores are issued, so
// they arrive while the stores drain (a wave's memory operations retire in
// issue order, so loads issued after the stores would wait for them).  gamma
// and beta stay in registers for all the rows.
__global__ void __launch_bounds__(SP_THREADS) sp_ln_fwd_pipe_kernel(SpArgs a) {
  __shared__ float red[4];
  const int h = (int)a.h;
  int64_t r = blockIdx.x;
  if (r >= a.n) return;
  u32x4 gw[SP_VPT], bw[SP_VPT], yw[SP_VPT], xw[SP_VPT];
  uint2 mw[SP_VPT];
  auto fetch = [&](int64_t row) {
#pragma unroll
    for (int i = 0; i < SP_VPT; ++i) {
      yw[i] = raw8_nt(a.y + row * a.h, col_of<true>(i, 0), h);
      xw[i] = raw8_nt(a.x + row * a.h, col_of<true>(i, 0), h);
      mw[i] = rawmask8_nt(a.mask + row * a.h, col_of<true>(i, 0), h);
    }
  };
#pragma unroll
  for (int i = 0; i < SP_VPT; ++i) {
    gw[i] = raw8<true>(a.gamma, i, h);
    bw[i] = raw8<true>(a.beta, i, h);
  }
  fetch(r);
  for (; r < a.n; r += gridDim.x) {
    float u[SP_VPT][8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < SP_VPT; ++i) {
      float yv[8], xv[8];
      unpack8(yw[i], yv);
      unpack8(xw[i], xv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        u[i][q] = fmaf(yv[q] * mask_at(mw[i], q), a.keep, xv[q]);
        s += u[i][q];
      }
    }
    const int64_t nr = r + gridDim.x;
    if (nr < a.n) fetch(nr);  // in flight during the reductions and this row's stores
    const float mean = block_sum(s, red) / (float)h;
    float v2 = 0.f;
#pragma unroll
    for (int i = 0; i < SP_VPT; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = col_of<true>(i, q) < h;
        const float d = u[i][q] - mean;
        v2 += in ? d * d : 0.f;
      }
    const float var = block_sum(v2, red) / (float)h;
    const float rstd = 1.f / sqrtf(var + a.eps);
    uint16_t *ur = a.uo + r * a.h, *zr = a.z + r * a.h;
#pragma unroll
    for (int i = 0; i < SP_VPT; ++i) {
      float zv[8], gv[8], bv[8];
      unpack8(gw[i], gv);
      unpack8(bw[i], bv);
#pragma unroll
      for (int q = 0; q < 8; ++q) zv[q] = fmaf((u[i][q] - mean) * rstd, gv[q], bv[q]);
      store8<true>(ur, i, h, u[i]);
      store8<true>(zr, i, h, zv);
    }
    if (threadIdx.x == 0) {
      a.mean[r] = mean;
      a.rstd[r] = rstd;
    }
  }
}

template <bool VEC, int NP>
__global__ void __launch_bounds__(SP_THREADS) sp_ln_bwd_kernel(SpArgs a) {
  __shared__ float red[4];
  const int h = (int)a.h;
  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    const float mean = a.mean[r], rstd = a.rstd[r];
    // every load of the row is issued before the first reduction
    float xh[NP * SP_VPT][8], g[NP * SP_VPT][8];
    u32x4 dnw[NP * SP_VPT];
    uint2 mw[NP * SP_VPT];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < NP * SP_VPT; ++i) {
      float uv[8], dzv[8], gv[8];
      load8<VEC>(a.u + r * a.h, i, h, uv);
      load8<VEC>(a.dz + r * a.h, i, h, dzv);
      load8<VEC>(a.gamma, i, h, gv);
      dnw[i] = raw8<VEC>(a.dun + r * a.h, i, h);
      mw[i] = rawmask8<VEC>(a.mask + r * a.h, i, h);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = col_of<VEC>(i, q) < h;
        xh[i][q] = in ? (uv[q] - mean) * rstd : 0.f;
        g[i][q] = dzv[q] * gv[q];
        sg += g[i][q];
        sgx += g[i][q] * xh[i][q];
      }
    }
    const float mg = block_sum(sg, red) / (float)h;
    const float mgx = block_sum(sgx, red) / (float)h;
#pragma unroll
    for (int i = 0; i < NP * SP_VPT; ++i) {
      float dxv[8], dyv[8], dn[8];
      unpack8(dnw[i], dn);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        dxv[q] = fmaf(rstd, g[i][q] - mg - xh[i][q] * mgx, dn[q]);
        dyv[q] = dxv[q] * mask_at(mw[i], q) * a.keep;
      }
      store8<VEC>(a.dx + r * a.h, i, h, dxv);
      store8<VEC>(a.dy + r * a.h, i, h, dyv);
    }
  }
}

// The backward for rows of up to 8192 columns (16-byte vectors): every workgroup
// (512 threads, two 8-element vectors of the row each) takes rows blockIdx.x,
// blockIdx.x + G, ... (G = gridDim.x), issues the next row's loads before this
// row's reductions and stores, and keeps its running dgamma / dbeta column sums
// (its rows in increasing order) in registers; it writes them once, as partial
// sums, at the end: part[blockIdx.x][2][h], or with BLOCKED (h a multiple of
// 64) part[2][h/64][gridDim.x][64], so that the reduction of one 64-column
// block reads one contiguous run.
constexpr int SP_BWD_WGS = 256;    // workgroups of the pipelined backward (one per CU)
constexpr int SP_BWD_THREADS = 512;
constexpr int SP_BWD_VPT = 2;      // 2 x 8 x 512 = 8192 columns
template <bool BLOCKED>
__global__ void __launch_bounds__(SP_BWD_THREADS) sp_ln_bwd_pipe_kernel(SpArgs a) {
  __shared__ float red[8];
  const int h = (int)a.h;
  const int tid = threadIdx.x;
  auto col = [&](int i) { return 8 * (tid + SP_BWD_THREADS * i); };
  auto sum = [&](float v) {  // over the workgroup, every thread gets the total
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
  };
  auto raw = [&](const uint16_t *row, int i) {
    const int c = col(i);
    return c < h ? *(const u32x4 *)(row + c) : u32x4{0u, 0u, 0u, 0u};
  };
  float pg[SP_BWD_VPT][8], pb[SP_BWD_VPT][8];
#pragma unroll
  for (int i = 0; i < SP_BWD_VPT; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) pg[i][q] = pb[i][q] = 0.f;
  u32x4 gw[SP_BWD_VPT], uw[SP_BWD_VPT], zw[SP_BWD_VPT], nw[SP_BWD_VPT];
  uint2 mw[SP_BWD_VPT];
  float mean = 0.f, rstd = 0.f;
  auto fetch = [&](int64_t row) {
#pragma unroll
    for (int i = 0; i < SP_BWD_VPT; ++i) {
      uw[i] = raw(a.u + row * a.h, i);
      zw[i] = raw(a.dz + row * a.h, i);
      nw[i] = raw(a.dun + row * a.h, i);
      const int c = col(i);
      mw[i] = c < h ? *(const uint2 *)(a.mask + row * a.h + c) : make_uint2(0u, 0u);
    }
    mean = a.mean[row];
    rstd = a.rstd[row];
  };
#pragma unroll
  for (int i = 0; i < SP_BWD_VPT; ++i) gw[i] = raw(a.gamma, i);
  int64_t r = blockIdx.x;
  if (r < a.n) fetch(r);
  for (; r < a.n; r += gridDim.x) {
    float xh[SP_BWD_VPT][8], g[SP_BWD_VPT][8];
    float sg = 0.f, sgx = 0.f;
    const float rm = mean, rr = rstd;
#pragma unroll
    for (int i = 0; i < SP_BWD_VPT; ++i) {
      float uv[8], dzv[8], gv[8];
      unpack8(uw[i], uv);
      unpack8(zw[i], dzv);
      unpack8(gw[i], gv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = col(i) + q < h;
        xh[i][q] = in ? (uv[q] - rm) * rr : 0.f;
        g[i][q] = dzv[q] * gv[q];
        sg += g[i][q];
        sgx += g[i][q] * xh[i][q];
        pg[i][q] = fmaf(dzv[q], xh[i][q], pg[i][q]);
        pb[i][q] += dzv[q];
      }
    }
    u32x4 dn[SP_BWD_VPT];
    uint2 mk[SP_BWD_VPT];
#pragma unroll
    for (int i = 0; i < SP_BWD_VPT; ++i) {
      dn[i] = nw[i];
      mk[i] = mw[i];
    }
    const int64_t nr = r + gridDim.x;
    if (nr < a.n) fetch(nr);  // in flight during the reductions and this row's stores
    const float mg = sum(sg) / (float)h;
    const float mgx = sum(sgx) / (float)h;
#pragma unroll
    for (int i = 0; i < SP_BWD_VPT; ++i) {
      float dxv[8], dyv[8], dnv[8];
      unpack8(dn[i], dnv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        dxv[q] = fmaf(rr, g[i][q] - mg - xh[i][q] * mgx, dnv[q]);
        dyv[q] = dxv[q] * mask_at(mk[i], q) * a.keep;
      }
      const int c = col(i);
      if (c < h) {
        *(u32x4 *)(a.dx + r * a.h + c) = pack8(dxv);
        *(u32x4 *)(a.dy + r * a.h + c) = pack8(dyv);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SP_BWD_VPT; ++i) {
    const int c = col(i);
    if (c < h) {
      float *qg, *qb;
      if constexpr (BLOCKED) {
        const int64_t nb = h / 64, blk = ((int64_t)(c >> 6) * gridDim.x + blockIdx.x) * 64 + (c & 63);
        qg = a.part + blk;
        qb = a.part + nb * gridDim.x * 64 + blk;
      } else {
        qg = a.part + (int64_t)blockIdx.x * 2 * a.h + c;
        qb = qg + a.h;
      }
      *(float4 *)qg = make_float4(pg[i][0], pg[i][1], pg[i][2], pg[i][3]);
      *(float4 *)(qg + 4) = make_float4(pg[i][4], pg[i][5], pg[i][6], pg[i][7]);
      *(float4 *)qb = make_float4(pb[i][0], pb[i][1], pb[i][2], pb[i][3]);
      *(float4 *)(qb + 4) = make_float4(pb[i][4], pb[i][5], pb[i][6], pb[i][7]);
    }
  }
}

// dgamma / dbeta partial column sums over one chunk of SP_RCHUNK rows (rows in
// increasing order): thread i of the grid's x dimension owns columns 8i .. 8i+7.
constexpr int SP_RCHUNK = 16;
constexpr int SP_PIPE_WGS = 512;  // workgroups of the pipelined row kernel (two per CU)
__global__ void __launch_bounds__(256) sp_ln_param_partial_kernel(SpArgs a) {
  const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c0 >= a.h) return;
  const int64_t r0 = (int64_t)blockIdx.y * SP_RCHUNK, r1 = min(a.n, r0 + SP_RCHUNK);
  float pg[8], pb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) pg[q] = pb[q] = 0.f;
  const bool full = c0 + 8 <= a.h && (a.h & 7) == 0;
  if (full && r1 - r0 == SP_RCHUNK) {
    // a whole chunk: all 2 x 16 loads in flight at once, then the fixed-order sums
    u32x4 uw[SP_RCHUNK], dw[SP_RCHUNK];
#pragma unroll
    for (int j = 0; j < SP_RCHUNK; ++j) {
      uw[j] = *(const u32x4 *)(a.u + (r0 + j) * a.h + c0);
      dw[j] = *(const u32x4 *)(a.dz + (r0 + j) * a.h + c0);
    }
#pragma unroll
    for (int j = 0; j < SP_RCHUNK; ++j) {
      const float mean = a.mean[r0 + j], rstd = a.rstd[r0 + j];
      float uv[8], dzv[8];
      unpack8(uw[j], uv);
      unpack8(dw[j], dzv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        pg[q] = fmaf(dzv[q], (uv[q] - mean) * rstd, pg[q]);
        pb[q] += dzv[q];
      }
    }
  } else {
#pragma unroll 4
  for (int64_t r = r0; r < r1; ++r) {
    const float mean = a.mean[r], rstd = a.rstd[r];
    float uv[8], dzv[8];
    if (full) {
      unpack8(*(const u32x4 *)(a.u + r * a.h + c0), uv);
      unpack8(*(const u32x4 *)(a.dz + r * a.h + c0), dzv);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = c0 + q < a.h;
        uv[q] = in ? bf2f(a.u[r * a.h + c0 + q]) : 0.f;
        dzv[q] = in ? bf2f(a.dz[r * a.h + c0 + q]) : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      pg[q] = fmaf(dzv[q], (uv[q] - mean) * rstd, pg[q]);
      pb[q] += dzv[q];
    }
  }
  }
  float *pr = a.part + (int64_t)blockIdx.y * 2 * a.h;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (c0 + q < a.h) {
      pr[c0 + q] = pg[q];
      pr[a.h + c0 + q] = pb[q];
    }
}

// dgamma[c], dbeta[c] = sum over the partials in workgroup order
__global__ void __launch_bounds__(256) sp_ln_param_reduce_kernel(const float *__restrict__ part, int nparts,
                                                                 int64_t h, uint16_t *__restrict__ dgamma,
                                                                 uint16_t *__restrict__ dbeta) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < h; c += (int64_t)gridDim.x * blockDim.x) {
    float sg = 0.f, sb = 0.f;
#pragma unroll 16
    for (int k = 0; k < nparts; ++k) {
      sg += part[(int64_t)k * 2 * h + c];
      sb += part[(int64_t)k * 2 * h + h + c];
    }
    dgamma[c] = f2bf(sg);
    dbeta[c] = f2bf(sb);
  }
}

// The same sums over the BLOCKED layout: workgroup (b, y) reduces columns
// 64b .. 64b+63 of dgamma (y = 0) or dbeta (y = 1); wave j adds partials
// j*per .. (j+1)*per-1 in increasing order (each of its loads is 64
// consecutive floats, the wave's run contiguous), then the 4 wave sums are
// added in wave order.
__global__ void __launch_bounds__(256) sp_ln_param_reduce_blocked_kernel(const float *__restrict__ part, int nparts,
                                                                         int64_t h, uint16_t *__restrict__ dgamma,
                                                                         uint16_t *__restrict__ dbeta) {
  __shared__ float acc[4][64];
  const int ci = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int per = (nparts + 3) / 4, k0 = min(nparts, j * per), k1 = min(nparts, k0 + per);
  const int64_t nb = h / 64;
  const float *p = part + ((int64_t)blockIdx.y * nb + blockIdx.x) * nparts * 64 + ci;
  float v = 0.f;
#pragma unroll 8
  for (int k = k0; k < k1; ++k) v += p[(int64_t)k * 64];
  acc[j][ci] = v;
  __syncthreads();
  if (j == 0) {
    const float t = (acc[0][ci] + acc[1][ci]) + (acc[2][ci] + acc[3][ci]);
    (blockIdx.y ? dbeta : dgamma)[(int64_t)blockIdx.x * 64 + ci] = f2bf(t);
  }
}

template <int NP>
hipError_t launch_fwd(const SpArgs &a, bool vec, hipStream_t st) {
  if (NP == 1 && vec) {  // several rows per workgroup, pipelined
    const unsigned grid = (unsigned)(a.n < SP_PIPE_WGS ? a.n : SP_PIPE_WGS);
    hipLaunchKernelGGL(sp_ln_fwd_pipe_kernel, dim3(grid), dim3(SP_THREADS), 0, st, a);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)(a.n < 1048576 ? a.n : 1048576);
  if (vec) hipLaunchKernelGGL((sp_ln_fwd_kernel<true, NP>), dim3(grid), dim3(SP_THREADS), 0, st, a);
  else hipLaunchKernelGGL((sp_ln_fwd_kernel<false, NP>), dim3(grid), dim3(SP_THREADS), 0, st, a);
  return hipGetLastError();
}
template <int NP>
hipError_t launch_bwd(const SpArgs &a, bool vec, hipStream_t st) {
  const unsigned grid = (unsigned)(a.n < 1048576 ? a.n : 1048576);
  if (vec) hipLaunchKernelGGL((sp_ln_bwd_kernel<true, NP>), dim3(grid), dim3(SP_THREADS), 0, st, a);
  else hipLaunchKernelGGL((sp_ln_bwd_kernel<false, NP>), dim3(grid), dim3(SP_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int tp_sp_ln_passes(int64_t h) { return (int)((h + SP_VPT * 8 * SP_THREADS - 1) / (SP_VPT * 8 * SP_THREADS)); }

// the pipelined backward serves rows of up to 8192 columns in 16-byte vectors
static bool sp_bwd_pipe(int64_t n, int64_t h) { return n > 0 && h % 8 == 0 && tp_sp_ln_passes(h) == 1; }

int tp_sp_ln_bwd_grid(int64_t n, int64_t h) {
  if (sp_bwd_pipe(n, h)) return (int)(n < SP_BWD_WGS ? n : SP_BWD_WGS);
  const int64_t chunks = (n + SP_RCHUNK - 1) / SP_RCHUNK;
  return (int)(chunks > 0 ? chunks : 1);
}

hipError_t tp_launch_sp_ln_fwd(int64_t n, int64_t h, float keep, float eps, const void *y, const void *x,
                               const uint8_t *mask, const void *gamma, const void *beta, void *u, void *z,
                               float *mean, float *rstd, hipStream_t st) {
  if (n == 0 || h == 0) return hipSuccess;
  SpArgs a = {};
  a.n = n;
  a.h = h;
  a.keep = keep;
  a.eps = eps;
  a.y = (const uint16_t *)y;
  a.x = (const uint16_t *)x;
  a.mask = mask;
  a.gamma = (const uint16_t *)gamma;
  a.beta = (const uint16_t *)beta;
  a.uo = (uint16_t *)u;
  a.z = (uint16_t *)z;
  a.mean = mean;
  a.rstd = rstd;
  const bool vec = h % 8 == 0;
  switch (tp_sp_ln_passes(h)) {
  case 1: return launch_fwd<1>(a, vec, st);
  case 2: return launch_fwd<2>(a, vec, st);
  default: return hipErrorInvalidValue;
  }
}

hipError_t tp_launch_sp_ln_bwd(int64_t n, int64_t h, float keep, const void *dz, const void *dun, const void *u,
                               const float *mean, const float *rstd, const void *gamma, const uint8_t *mask,
                               void *dx, void *dy, void *dgamma, void *dbeta, float *part, hipStream_t st) {
  if (h == 0) return hipSuccess;
  SpArgs a = {};
  a.n = n;
  a.h = h;
  a.keep = keep;
  a.dz = (const uint16_t *)dz;
  a.dun = (const uint16_t *)dun;
  a.u = (const uint16_t *)u;
  a.mean = const_cast<float *>(mean);
  a.rstd = const_cast<float *>(rstd);
  a.gamma = (const uint16_t *)gamma;
  a.mask = mask;
  a.dx = (uint16_t *)dx;
  a.dy = (uint16_t *)dy;
  a.part = part;
  const bool vec = h % 8 == 0;
  const int chunks = tp_sp_ln_bwd_grid(n, h);
  hipError_t e = hipSuccess;
  if (sp_bwd_pipe(n, h)) {
    // rows, and their partial column sums, in one kernel; then the fixed-order reduction
    if (h % 64 == 0) {
      hipLaunchKernelGGL(sp_ln_bwd_pipe_kernel<true>, dim3((unsigned)chunks), dim3(SP_BWD_THREADS), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(sp_ln_param_reduce_blocked_kernel, dim3((unsigned)(h / 64), 2), dim3(256), 0, st, part,
                         chunks, h, (uint16_t *)dgamma, (uint16_t *)dbeta);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(sp_ln_bwd_pipe_kernel<false>, dim3((unsigned)chunks), dim3(SP_BWD_THREADS), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t rb = (h + 255) / 256;
    hipLaunchKernelGGL(sp_ln_param_reduce_kernel, dim3((unsigned)(rb < 65536 ? rb : 65536)), dim3(256), 0, st,
                       part, chunks, h, (uint16_t *)dgamma, (uint16_t *)dbeta);
    return hipGetLastError();
  }
  if (n > 0) {
    switch (tp_sp_ln_passes(h)) {
    case 1: e = launch_bwd<1>(a, vec, st); break;
    case 2: e = launch_bwd<2>(a, vec, st); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  const int64_t cb = (h + 8 * 256 - 1) / (8 * 256);
  hipLaunchKernelGGL(sp_ln_param_partial_kernel, dim3((unsigned)cb, (unsigned)chunks), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rb = (h + 255) / 256;
  hipLaunchKernelGGL(sp_ln_param_reduce_kernel, dim3((unsigned)(rb < 65536 ? rb : 65536)), dim3(256), 0, st, part,
                     chunks, h, (uint16_t *)dgamma, (uint16_t *)dbeta);
  return hipGetLastError();
}
