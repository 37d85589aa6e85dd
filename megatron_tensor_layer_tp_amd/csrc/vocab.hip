// vocab.hip -- vocab-parallel cross-entropy statistics and embedding gather.
//
// Cross entropy split by vocab (lecture 16 notes §5.5; book "7.3 模型并行与张
// 量并行" §7.3.4): each shard reduces its own [s, V/t] logit slice to three
// numbers per position -- the row max, the sum of exp(z - max) and the target's
// logit when the target id falls in the shard -- so only 3 scalars per token
// ever leave the device instead of the logits.
//
// The embedding split by vocab returns the table row for ids inside the
// shard and a zero vector otherwise; summing over shards restores the lookup.
//
// Both are HBM-streaming kernels.  The CE kernel gives each row to one
// 256-thread workgroup which issues all of its 16-byte loads for the row up
// front (16 per thread covers a 16384-float row), takes the exact row max,
// then sums exp(z - max) from registers: the logits are read from HBM once.
// The logits are read, and the CE gradient written, with non-temporal
// accesses: each byte is touched once, and keeping it out of the caches keeps
// their dirty lines from being written back under the next kernel.
#include "launch.h"

namespace {

constexpr int CE_THREADS = 256;
constexpr int CE_PER = 16;  // 16-byte vectors held per thread per pass
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// VW = 4: rows are 16-byte aligned (Vs % 4 == 0); VW = 1: any Vs.
template <int VW>
__global__ void __launch_bounds__(CE_THREADS) vocab_ce_kernel(const float *__restrict__ z,
                                                              const int64_t *__restrict__ tgt,
                                                              int64_t s, int64_t Vs, int64_t start,
                                                              float *__restrict__ m_out,
                                                              float *__restrict__ se_out,
                                                              float *__restrict__ tl_out) {
  typedef float vec_t __attribute__((ext_vector_type(VW)));
  __shared__ float red[CE_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t nvec = Vs / VW;
  for (int64_t row = blockIdx.x; row < s; row += gridDim.x) {
    const vec_t *p = (const vec_t *)(z + row * Vs);
    float run_m = -INFINITY, run_s = 0.f;
    for (int64_t base = 0; base < nvec; base += (int64_t)CE_THREADS * CE_PER) {
      vec_t v[CE_PER];
#pragma unroll
      for (int i = 0; i < CE_PER; ++i) {
        const int64_t idx = base + tid + (int64_t)CE_THREADS * i;
        if (idx < nvec) v[i] = __builtin_nontemporal_load(p + idx);
        else
#pragma unroll
          for (int e = 0; e < VW; ++e) v[i][e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < CE_PER; ++i)
#pragma unroll
        for (int e = 0; e < VW; ++e) mx = fmaxf(mx, v[i][e]);
      mx = wave_max(mx);
      if (lane == 0) red[wid] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();
      const float new_m = fmaxf(run_m, mx);
      float sum = 0.f;
      if (new_m != -INFINITY) {
        const float mb = new_m * LOG2E;
#pragma unroll
        for (int i = 0; i < CE_PER; ++i)
#pragma unroll
          for (int e = 0; e < VW; ++e) sum += exp2f(fmaf(v[i][e], LOG2E, -mb));
      }
      sum = wave_sum(sum);
      if (lane == 0) red[wid] = sum;
      __syncthreads();
      sum = (red[0] + red[1]) + (red[2] + red[3]);
      __syncthreads();
      // rescale the running sum when a later pass raises the max (rows > 16384 floats)
      run_s = (run_s == 0.f ? 0.f : run_s * exp2f((run_m - new_m) * LOG2E)) + sum;
      run_m = new_m;
    }
    if (tid == 0) {
      const int64_t y = tgt[row];
      m_out[row] = run_m;
      se_out[row] = run_s;
      tl_out[row] = (y >= start && y - start < Vs) ? z[row * Vs + (y - start)] : 0.f;
    }
  }
}

// Gradient of the cross entropy with respect to one shard's logit slice
// (lecture 16 notes §5.5: each shard differentiates its own slice once the
// combined max M and sum S are known):
//     dz[r,j] = g[r] * (exp(z[r,j] - M[r]) / S[r] - [start + j == target[r]]).
// One workgroup per row streams the row once: 16-byte loads and stores (VW =
// 4), fp32 or bf16 output.
template <int VW, bool BF16_OUT>
__global__ void __launch_bounds__(CE_THREADS) vocab_ce_bwd_kernel(const float *__restrict__ z,
                                                                  const int64_t *__restrict__ tgt,
                                                                  const float *__restrict__ Mg,
                                                                  const float *__restrict__ Sg,
                                                                  const float *__restrict__ g, int64_t s,
                                                                  int64_t Vs, int64_t start,
                                                                  void *__restrict__ out) {
  typedef float vec_t __attribute__((ext_vector_type(VW)));
  const int64_t nvec = Vs / VW;
  for (int64_t row = blockIdx.x; row < s; row += gridDim.x) {
    const float mb = Mg[row] * LOG2E;
    const float gr = g[row];
    const float scale = gr / Sg[row];
    const int64_t y = tgt[row] - start;  // target column; outside [0, Vs) when not in the shard
    const vec_t *p = (const vec_t *)(z + row * Vs);
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < nvec; i += CE_THREADS) {
      const vec_t v = __builtin_nontemporal_load(p + i);
      float o[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        o[e] = exp2f(fmaf(v[e], LOG2E, -mb)) * scale;
        if (i * VW + e == y) o[e] -= gr;
      }
      if constexpr (BF16_OUT) {
        uint16_t *dst = (uint16_t *)out + row * Vs + i * VW;
        if constexpr (VW == 4) {
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          const f2 lo = {o[0], o[1]}, hi = {o[2], o[3]};
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          const u2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, b2)),
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, b2))};
          __builtin_nontemporal_store(w, (u2 *)dst);
        } else {
          dst[0] = __builtin_bit_cast(uint16_t, (__bf16)o[0]);
        }
      } else {
        vec_t w;
#pragma unroll
        for (int e = 0; e < VW; ++e) w[e] = o[e];
        __builtin_nontemporal_store(w, (vec_t *)((float *)out + row * Vs) + i);
      }
    }
  }
}

// Merge the per-tile-column statistics of the fused LM-head GEMM into the
// shard's three numbers per position.  ws holds P parts per row, part-major:
// ws[p][row] = the max over tile column p, ws[P + p][row] = the sum of
// exp(z - that max), and ws[2P][row] = the target's logit (written by the
// tile that holds column target - start).  A workgroup takes 64 rows, one per
// lane, so every load is a run of 64 consecutive floats; its 4 waves split the
// parts (wave q: p = q, q + 4, ...) and their results combine in wave order:
// M = max_p m_p, S = sum_p se_p exp(m_p - M).  Up to 4 * 16 parts per row all
// loads of a thread are in flight at once (one memory round trip).
__global__ void __launch_bounds__(256) ce_merge_kernel(const float *__restrict__ ws, int P, int64_t s,
                                                       int64_t Vs, int64_t start,
                                                       const int64_t *__restrict__ tgt,
                                                       float *__restrict__ m_out, float *__restrict__ se_out,
                                                       float *__restrict__ tl_out) {
  constexpr int U = 16;
  __shared__ float part[2][4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 64 + lane;
  const bool live = row < s;
  const float *wm = ws + row, *wse = ws + (int64_t)P * s + row;
  float mv[U], sv[U];
  float mx = -INFINITY;
  if (P <= 4 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = q + 4 * u;
      const bool ok = live && p < P;
      mv[u] = ok ? wm[(int64_t)p * s] : -INFINITY;
      sv[u] = ok ? wse[(int64_t)p * s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, mv[u]);
  } else if (live) {
    for (int p = q; p < P; p += 4) mx = fmaxf(mx, wm[(int64_t)p * s]);
  }
  part[0][q][lane] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(part[0][0][lane], part[0][1][lane]), fmaxf(part[0][2][lane], part[0][3][lane]));
  float sum = 0.f;
  if (live && M != -INFINITY) {
    const float mb = M * LOG2E;
    if (P <= 4 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (mv[u] != -INFINITY) sum += sv[u] * exp2f(fmaf(mv[u], LOG2E, -mb));
    } else {
      for (int p = q; p < P; p += 4) {
        const float mp = wm[(int64_t)p * s];
        if (mp != -INFINITY) sum += wse[(int64_t)p * s] * exp2f(fmaf(mp, LOG2E, -mb));
      }
    }
  }
  part[1][q][lane] = sum;
  __syncthreads();
  if (q == 0 && live) {
    const int64_t y = tgt[row];
    m_out[row] = M;
    se_out[row] = ((part[1][0][lane] + part[1][1][lane]) + part[1][2][lane]) + part[1][3][lane];
    tl_out[row] = (y >= start && y - start < Vs) ? ws[(int64_t)2 * P * s + row] : 0.f;
  }
}

// One workgroup per output row: copy the owned table row, or write zeros.
template <typename T>
__global__ void __launch_bounds__(256) vocab_embed_kernel(int64_t n, int64_t Vs, int64_t nelem,
                                                          int64_t start,
                                                          const int64_t *__restrict__ ids,
                                                          const T *__restrict__ table,
                                                          T *__restrict__ out) {
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int64_t id = ids[r];
    const bool in = id >= start && id - start < Vs;
    T *dst = out + r * nelem;
    if (in) {
      const T *src = table + (id - start) * nelem;
      for (int64_t i = threadIdx.x; i < nelem; i += blockDim.x) dst[i] = src[i];
    } else {
      T zero;
      __builtin_memset(&zero, 0, sizeof(T));
      for (int64_t i = threadIdx.x; i < nelem; i += blockDim.x) dst[i] = zero;
    }
  }
}

}  // namespace

hipError_t tp_launch_vocab_ce(int64_t s, int64_t Vs, int64_t start, const float *z, const int64_t *tgt,
                              float *m, float *se, float *tl, hipStream_t st) {
  if (s == 0) return hipSuccess;
  const unsigned grid = (unsigned)(s < 1048576 ? s : 1048576);
  const bool v4 = (Vs % 4 == 0) && (((uintptr_t)z & 15) == 0);
  if (v4)
    hipLaunchKernelGGL(vocab_ce_kernel<4>, dim3(grid), dim3(CE_THREADS), 0, st, z, tgt, s, Vs, start, m, se, tl);
  else
    hipLaunchKernelGGL(vocab_ce_kernel<1>, dim3(grid), dim3(CE_THREADS), 0, st, z, tgt, s, Vs, start, m, se, tl);
  return hipGetLastError();
}

hipError_t tp_launch_ce_merge(const float *ws, int P, int64_t s, int64_t Vs, int64_t start, const int64_t *tgt,
                              float *m, float *se, float *tl, hipStream_t st) {
  if (s == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_merge_kernel, dim3((unsigned)((s + 63) / 64)), dim3(256), 0, st, ws, P, s, Vs, start, tgt,
                     m, se, tl);
  return hipGetLastError();
}

hipError_t tp_launch_vocab_ce_bwd(bool bf16_out, int64_t s, int64_t Vs, int64_t start, const float *z,
                                  const int64_t *tgt, const float *M, const float *S, const float *g, void *out,
                                  hipStream_t st) {
  if (s == 0 || Vs == 0) return hipSuccess;
  const unsigned grid = (unsigned)(s < 1048576 ? s : 1048576);
  const bool v4 = Vs % 4 == 0 && (((uintptr_t)z | (uintptr_t)out) & 15) == 0;
  const dim3 b(CE_THREADS);
  if (v4 && bf16_out)
    hipLaunchKernelGGL((vocab_ce_bwd_kernel<4, true>), dim3(grid), b, 0, st, z, tgt, M, S, g, s, Vs, start, out);
  else if (v4)
    hipLaunchKernelGGL((vocab_ce_bwd_kernel<4, false>), dim3(grid), b, 0, st, z, tgt, M, S, g, s, Vs, start, out);
  else if (bf16_out)
    hipLaunchKernelGGL((vocab_ce_bwd_kernel<1, true>), dim3(grid), b, 0, st, z, tgt, M, S, g, s, Vs, start, out);
  else
    hipLaunchKernelGGL((vocab_ce_bwd_kernel<1, false>), dim3(grid), b, 0, st, z, tgt, M, S, g, s, Vs, start, out);
  return hipGetLastError();
}

hipError_t tp_launch_vocab_embed(int elem_bytes, int64_t n, int64_t Vs, int64_t h, int64_t start,
                                 const int64_t *ids, const void *table, void *out, hipStream_t st) {
  if (n == 0 || h == 0) return hipSuccess;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t bytes = h * elem_bytes;
  const unsigned grid = (unsigned)(n < 1048576 ? n : 1048576);
  const bool aligned = (((uintptr_t)table | (uintptr_t)out) & 15) == 0;
  if (aligned && bytes % 16 == 0)
    hipLaunchKernelGGL(vocab_embed_kernel<u32x4>, dim3(grid), dim3(256), 0, st, n, Vs, bytes / 16, start, ids,
                       (const u32x4 *)table, (u32x4 *)out);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(vocab_embed_kernel<uint32_t>, dim3(grid), dim3(256), 0, st, n, Vs, h, start, ids,
                       (const uint32_t *)table, (uint32_t *)out);
  else
    hipLaunchKernelGGL(vocab_embed_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, n, Vs, h, start, ids,
                       (const uint16_t *)table, (uint16_t *)out);
  return hipGetLastError();
}
