// gemm_bf16_kernels.h -- bf16 MFMA GEMM kernels for gfx950 (CDNA4) with
// fused epilogues; included by the launch translation units (single products
// and paired products), each instantiating the variants it launches.
//
// Every matrix product of the shard (MLP, SwiGLU, attention projections, LM
// head; forward and backward) runs through these kernel templates.  The
// products are the column- and row-parallel GEMMs of the pages (book "7.3 模型
// 并行与张量并行" §7.3.2-§7.3.4, lecture 16 notes §5.2-§5.5); the element-wise
// activation, its derivative and the SwiGLU gating run in the epilogue, so the
// [s, f/t] intermediates are written once and read once.
//
// Design (MI355X first):
//  * 256 threads = 4 wave64s in a 2x2 grid; a workgroup computes a BMxBN tile,
//    each wave a (BM/2)x(BN/2) sub-tile of 32x32 v_mfma_f32_32x32x16_bf16 blocks
//    accumulated in fp32.
//  * K advances 64 at a time through two LDS stages: the next tile's loads are
//    in flight while the MFMAs consume the current stage, one barrier per step.
//  * Main path (16-byte-aligned operands): buffer loads write straight into
//    LDS (no register staging).  k-contiguous operands sit in LDS as
//    [rows][64 k] with XOR-swizzled 16-byte chunks; m/n-contiguous operands
//    sit as [64 k][cols] and reach the MFMA layout through the LDS transpose
//    read (ds_read_b64_tr_b16).
//  * Fallback path (odd sizes or leading dimensions): element-wise loads
//    through registers, transposed in registers on the way to LDS.
//  * Workgroup ids are remapped so that consecutive tiles land on the same XCD
//    (each XCD has its own L2), then grouped along M for panel reuse.
#pragma once
#include <type_traits>

#include "gemm_desc.h"
#include "launch.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int NTHREADS = 256;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

__device__ __forceinline__ uint32_t elem16(const u32x4 &v, int i) {
  uint32_t w = v[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// ---------------------------------------------------------------------------
// Operand staging.  Every loader has the same interface:
//   init(ld, extent_left, tid)  per-thread offsets for a new operand / segment
//   load(tile, kleft, ...)      fetch one 64-deep K slice into registers
//   store(lds, tid)             write it to LDS as [rows][64 k], swizzled
// The 16-byte ("VEC") loaders use raw buffer loads: an out-of-range offset
// returns zeros, so ragged edges need no branches.
// ---------------------------------------------------------------------------
constexpr uint32_t OOB = 0x80000000u;       // offset past every buffer's end
constexpr int NREC = 0x7ffffff0;            // records (bytes) of every buffer
constexpr int RSRC_W3 = 0x00020000;         // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mkrsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, NREC, RSRC_W3);
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// k-contiguous operand, R rows x 64 k: thread t owns chunk (t & 7) of rows
// (t >> 3) + 32 i, R/32 chunks.
template <int R, bool VEC>
struct LoadKC {
  static constexpr int N = R / 32;
  u32x4 v[N];
  uint32_t off[N];   // VEC: byte offset of the chunk in the tile, OOB for rows past the edge
  int64_t ld;
  int rows_left, c;
  __device__ __forceinline__ void init(int64_t ld_, int rows_left_, int tid) {
    ld = ld_;
    rows_left = rows_left_;
    c = tid & 7;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int rl = (tid >> 3) + 32 * i;
      off[i] = rl < rows_left ? (uint32_t)(rl * ld * 2 + c * 16) : OOB;
    }
  }
  // tile = &Op[row0][k0]; kleft = valid k from k0 on
  __device__ __forceinline__ void load(const uint16_t *tile, int kleft, int tid) {
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t r = mkrsrc(tile);
      const bool kok = c * 8 < kleft;
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = bload(r, kok ? off[i] : OOB);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int rl = (tid >> 3) + 32 * i;
        u32x4 t = zero4();
        if (rl < rows_left) {
          const uint16_t *q = tile + (int64_t)rl * ld + c * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t x = (c * 8 + e < kleft) ? q[e] : 0u;
            t[e >> 1] |= (e & 1) ? (x << 16) : x;
          }
        }
        v[i] = t;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = (tid >> 3) + 32 * i;
      lds[r * 8 + (c ^ swz(r))] = v[i];
    }
  }
};

// Operand with the row index (m or n) contiguous in memory, stored [k][row]:
// a thread owns one 8x8 block (kb, rb), loads 8 k-rows of 8 consecutive
// elements and transposes them in registers so that LDS row rb*8+i holds 8
// consecutive k.  Threads 0-127 cover rows [0, R/2), threads 128-255 rows
// [R/2, R), so each wave reads from one source: with DUAL the upper half
// comes from a second matrix (SwiGLU up next to gate) at the same columns.
template <int R, bool VEC, bool DUAL>
struct LoadRC {
  static constexpr int H = R / 16;   // row blocks per half
  u32x4 v[8];
  uint32_t off0;    // VEC: byte offset of (k = 8 kb, col) in the tile, OOB if idle / past the edge
  uint32_t ld2;
  int64_t ld;
  int kb, rb, col, cols_left;
  bool active;
  __device__ __forceinline__ void init(int64_t ld_, int cols_left_, int tid) {
    ld = ld_;
    ld2 = (uint32_t)(ld_ * 2);
    cols_left = cols_left_;
    const int half = tid >> 7, u = tid & 127;
    rb = half * H + u % H;
    kb = u / H;
    active = kb < 8;
    col = DUAL ? (u % H) * 8 : rb * 8;   // column within the source matrix's tile
    off0 = (active && col < cols_left) ? (uint32_t)(kb * 8 * ld * 2 + col * 2) : OOB;
  }
  // tile = &Op[k0][col0] of this wave's source; kleft = valid k rows from k0
  __device__ __forceinline__ void load(const uint16_t *tile, int kleft, int tid) {
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t r = mkrsrc(tile);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = off0 != OOB && kb * 8 + e < kleft;
        v[e] = bload(r, ok ? off0 + e * ld2 : OOB);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x4 t = zero4();
        if (active && kb * 8 + e < kleft) {
          const uint16_t *q = tile + (int64_t)(kb * 8 + e) * ld + col;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            uint32_t x = (col + i < cols_left) ? q[i] : 0u;
            t[i >> 1] |= (i & 1) ? (x << 16) : x;
          }
        }
        v[e] = t;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = elem16(v[2 * q], i) | (elem16(v[2 * q + 1], i) << 16);
      const int r = rb * 8 + i;
      lds[r * 8 + (kb ^ swz(r))] = o;
    }
  }
};

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// 8 fp32 -> 8 bf16 with the hardware pair conversion (round to nearest even)
__device__ __forceinline__ u32x4 pack8(const float *v) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2_t p = {v[2 * q], v[2 * q + 1]};
    o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
  }
  return o;
}

// a run of 8 bf16 outputs; `nt` streams it past the caches (a non-temporal store)
__device__ __forceinline__ void st8(uint16_t *p, u32x4 v, bool nt) {
  if (nt) __builtin_nontemporal_store(v, (u32x4 *)p);
  else *(u32x4 *)p = v;
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
                                     const float *x, const float *u, const u32x4 *pre = nullptr) {
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
    // fp32 outputs (the LM head's logits) are streamed past the caches: they are read
    // back only by a later kernel, and dirty lines left in the Infinity Cache would be
    // written back while that kernel streams them in
    float *o = (float *)d.C[sc] + (int64_t)gm * d.ldc[sc] + gn;
    if (full) {
      const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
      __builtin_nontemporal_store(lo, (f32x4 *)o);
      __builtin_nontemporal_store(hi, (f32x4 *)(o + 4));
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
      if (full && pre != nullptr) {  // loaded ahead by the caller
        unpack8(pre[0], a0);
        if constexpr (EPI == EPI_SWIGLU_BWD) unpack8(pre[1], a1);
      } else if (full) {
        unpack8(*(const u32x4 *)((const uint16_t *)d.ai0 + o), a0);
        if constexpr (EPI == EPI_SWIGLU_BWD) unpack8(*(const u32x4 *)((const uint16_t *)d.ai1 + o), a1);
      } else {
        for (int q = 0; q < 8; ++q) {
          a0[q] = q < cnt ? tp_bf2f(((const uint16_t *)d.ai0)[o + q]) : 0.f;
          if constexpr (EPI == EPI_SWIGLU_BWD) a1[q] = q < cnt ? tp_bf2f(((const uint16_t *)d.ai1)[o + q]) : 0.f;
        }
      }
    }
    // the activation kind is uniform: branch once per run of 8 so that the 8
    // independent element chains interleave
    if constexpr (EPI == EPI_ACT_FWD) {
      if (d.act == ACT_GELU) {
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = tp_gelu(x[q]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = tp_relu(x[q]);
      }
    } else if constexpr (EPI == EPI_ACT_BWD) {
      if (d.act == ACT_GELU) {
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = x[q] * tp_gelu_grad(a0[q]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = x[q] * tp_relu_grad(a0[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if constexpr (EPI == EPI_STORE) {
        y[q] = x[q];
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
      st8(C, pack8(y), d.stream_out & 1);
      if constexpr (EPI == EPI_ACT_FWD || EPI == EPI_SWIGLU_FWD) {
        if (w_o0) st8(O0, pack8(x), d.stream_out & 2);
      }
      if constexpr (EPI == EPI_SWIGLU_FWD) st8(O1, pack8(u), d.stream_out & 4);
      if constexpr (EPI == EPI_SWIGLU_BWD) st8(O0, pack8(y2), d.stream_out & 2);
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

// Reductions over the LPR (8 or 16) consecutive lanes of a DPP row with DPP
// moves (VALU, no LDS round trip): xor 1 and xor 2 within quads, then the
// half-row and row mirrors; every lane of the group ends with the result.
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  if constexpr (LPR == 16)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  return v;
}
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  if constexpr (LPR == 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

// Cross-entropy statistics of the LM head's logits without storing them
// (lecture 16 notes §5.5, the fused vocab-parallel cross entropy): the LPR
// lanes holding row gm's columns of one wave's strip (8 each, from gn) reduce
// them to the row's max over the valid columns (mx) and the sum of
// exp(z - max) (se); every one of them gets both.  The lane holding the target
// id's column (if any; over the whole launch exactly one lane holds it)
// stores that logit to tl[gm], read back from the LDS strip src that x was
// loaded from (an index into x itself would put x in scratch memory).  Every
// lane must call it (cross-lane moves); rows >= M store nothing.
template <int LPR>
__device__ __forceinline__ void ce_row8(const GemmDesc &d, int gm, int gn, int nlen, const float *x,
                                        const float *src, float *tl, float &mx_out, float &se_out) {
  static_assert(LPR == 8 || LPR == 16, "row reductions span 8 or 16 lanes");
  constexpr float LOG2E = 1.4426950408889634f;
  const int nv = min(8, nlen - gn);  // valid columns of this lane (may be <= 0)
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (q < nv) mx = fmaxf(mx, x[q]);
  mx = row_max<LPR>(mx);
  float se = 0.f;
  if (mx != -INFINITY) {
    const float mb = mx * LOG2E;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < nv) se += tp_exp2(fmaf(x[q], LOG2E, -mb));
  }
  mx_out = mx;
  se_out = row_sum<LPR>(se);
  if (gm < d.M) {
    const int64_t j = ((const int64_t *)d.ai0)[gm] - d.vstart - gn;
    if (j >= 0 && j < nv) tl[gm] = src[j];
  }
}

// The NC wave columns' statistics of each of the tile's BM rows (red[j*BM + r]
// = max, red[(NC + j)*BM + r] = sum of exp(z - max), j = wave column) merged in
// column order -- M = max_j m_j, S = sum_j s_j exp(m_j - M), the combine the
// per-row merge across tiles repeats -- and stored as tile column tc's part:
// ws[tc][gm] = M, ws[P + tc][gm] = S (P = tiles_n, rows of length d.M), so a
// tile stores two runs of BM consecutive floats.  Every thread must call it
// (workgroup barrier).
template <int BM, int NC, int NT>
__device__ __forceinline__ void ce_tile_merge(const GemmDesc &d, const float *red, int m0, int tc) {
  static_assert(NT >= BM, "one thread per row of the tile");
  constexpr float LOG2E = 1.4426950408889634f;
  __syncthreads();
  const int t = threadIdx.x, gm = m0 + t;
  if (t < BM && gm < d.M) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NC; ++j) mx = fmaxf(mx, red[j * BM + t]);
    float se = 0.f;
    if (mx != -INFINITY) {
      const float mb = mx * LOG2E;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const float mj = red[j * BM + t];
        if (mj != -INFINITY) se += red[(NC + j) * BM + t] * tp_exp2(fmaf(mj, LOG2E, -mb));
      }
    }
    float *w = d.ws + (int64_t)tc * d.M + gm;
    w[0] = mx;
    w[(int64_t)d.tiles_n * d.M] = se;
  }
}

// ---------------------------------------------------------------------------
// Epilogue shared by both kernels.  Each wave stages one 32-row strip of its
// accumulators at a time through LDS (fp32, rows padded by 8 floats so the
// MFMA-layout writes of the two half-waves fall on different banks), then
// reads rows back as runs of 8 consecutive columns: the activation math runs
// once per element and every global access is 16 bytes wide.
// 32x32 accumulator layout: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
// column l%32 of the block.  `ep` is this wave's private strip (32 x (WTN+8)).
// All waves of the workgroup must call it (it holds workgroup barriers).
// ---------------------------------------------------------------------------
// fp32 outputs straight from the accumulator layout: a half-wave's 32 lanes hold
// 32 consecutive columns of one row, so each 4-byte store instruction writes two
// full 128-byte row segments; no LDS round trip and no workgroup barrier.  The
// stored outputs (fp32 C, e.g. logits) stream past the caches, since a later
// kernel reads them; split-K partials (PARTIAL) stay cacheable for the reduction.
template <int BM, int BN, int NW, bool PARTIAL>
__device__ __forceinline__ void epilogue_f32_direct(const GemmDesc &d, f32x16 (&acc)[BM / 64][2 * BN / NW / 32],
                                                    int lane, int wm, int wn, int m0, int n0, int nlen, int sc,
                                                    int split) {
  constexpr int WTM = BM / 2, WTN = BN / (NW / 2), FM = WTM / 32, FN = WTN / 32;
  float *C;
  int64_t ldc;
  int coff = 0;  // column of the tile's first output column in C
  if constexpr (PARTIAL) {
    C = d.ws + (int64_t)split * d.M * d.N;
    ldc = d.N;
    coff = d.kseg ? 0 : d.seg_col0[sc];
  } else {
    C = (float *)d.C[sc];
    ldc = d.ldc[sc];
  }
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int gn = n0 + wn * WTN + fn * 32 + (lane & 31);
    if (gn >= nlen) continue;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int r0 = m0 + wm * WTM + fm * 32 + rsub;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = r0 + 8 * (e >> 2) + (e & 3);
        if (gm >= d.M) continue;
        float *o = C + (int64_t)gm * ldc + coff + gn;
        if constexpr (PARTIAL) *o = acc[fm][fn][e];
        else __builtin_nontemporal_store(acc[fm][fn][e], o);
      }
    }
  }
}

template <int BM, int BN, int EPI, bool OUT_F32, bool VEC, bool DUAL, int NW = 4>
__device__ __forceinline__ void epilogue(const GemmDesc &d, f32x16 (&acc)[BM / 64][2 * BN / NW / 32], float *ep,
                                         int lane, int wm, int wn, int m0, int n0, int nlen, int sc, int split,
                                         float *red = nullptr) {
  constexpr int WTM = BM / 2, WTN = BN / (NW / 2), FM = WTM / 32, FN = WTN / 32;
  constexpr int EPS = WTN + 8;                      // strip row stride (floats)
  constexpr int OUTW = DUAL ? WTN / 2 : WTN;        // output columns per strip row
  constexpr int LPR = OUTW / 8;                     // lanes per strip row
  constexpr int RPI = 64 / LPR;                     // strip rows per pass
  constexpr int NIT = (32 + RPI - 1) / RPI;         // passes per 32-row strip
  // 96-column strips (192-wide tiles): 12 lanes per row, 5 rows per pass, lanes 60-63 idle
  static_assert(EPI != EPI_CE_STATS || (64 % LPR == 0 && 32 % RPI == 0), "CE rows span a DPP row");
  const int ci = lane & 31;
  const int rsub = 4 * (lane >> 5);
  const int col_base = n0 + (DUAL ? wn * (BN / NW) : wn * WTN);  // DUAL: BN/NW gate + as many up columns
  // epilogues that read inputs (Z, or G and U) issue this strip's loads before its
  // LDS round trip, so their latency runs under the barriers and LDS writes
  constexpr bool PRE = VEC && (EPI == EPI_ACT_BWD || EPI == EPI_SWIGLU_BWD);
  constexpr int NPRE = PRE ? NIT : 1;
  auto pass_at = [&](int fm, int it, int &gm, int &gn, bool &live, int &r, int &c) {
    const int r0 = it * RPI + lane / LPR;
    live = lane < RPI * LPR && r0 < 32;
    r = live ? r0 : 0;
    c = (lane % LPR) * 8;
    gm = m0 + wm * WTM + fm * 32 + r;
    gn = col_base + c;
  };
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    u32x4 pre[NPRE][2];
    if constexpr (PRE) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        int gm, gn, r, c;
        bool live;
        pass_at(fm, it, gm, gn, live, r, c);
        pre[it][0] = pre[it][1] = u32x4{0u, 0u, 0u, 0u};
        if (live && gm < d.M && gn + 8 <= nlen) {
          const int64_t o = (int64_t)gm * d.ldai + gn;
          pre[it][0] = *(const u32x4 *)((const uint16_t *)d.ai0 + o);
          if constexpr (EPI == EPI_SWIGLU_BWD) pre[it][1] = *(const u32x4 *)((const uint16_t *)d.ai1 + o);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ep[(8 * (e >> 2) + rsub + (e & 3)) * EPS + fn * 32 + ci] = acc[fm][fn][e];
    __syncthreads();
#pragma unroll PRE ? NIT : 2
    for (int it = 0; it < NIT; ++it) {
      const int r0 = it * RPI + lane / LPR;
      const bool live = lane < RPI * LPR && r0 < 32;
      const int r = live ? r0 : 0;
      const int c = (lane % LPR) * 8;
      const float *src = ep + r * EPS + c;
      float x[8], u[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = src[q];
      if constexpr (DUAL) {
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = src[OUTW + q];
      }
      const int gm = m0 + wm * WTM + fm * 32 + r;
      const int gn = col_base + c;
      if constexpr (EPI == EPI_CE_STATS) {
        // per row of the strip: this wave column's statistics into red (LDS)
        float mx, se;
        ce_row8<LPR>(d, gm, gn, nlen, x, src, d.ws + (int64_t)2 * d.tiles_n * d.M, mx, se);
        if (lane % LPR == 0) {
          const int rt = wm * WTM + fm * 32 + r;
          red[wn * BM + rt] = mx;
          red[(NW / 2 + wn) * BM + rt] = se;
        }
      } else {
        if (live && gm < d.M && gn < nlen)
          epi8<EPI, OUT_F32, VEC>(d, gm, gn, nlen, sc, split, x, u, PRE ? pre[PRE ? it : 0] : nullptr);
      }
    }
  }
  if constexpr (EPI == EPI_CE_STATS) ce_tile_merge<BM, NW / 2, 64 * NW>(d, red, m0, n0 / BN);
}

template <int BM, int BN>
struct Smem {
  u32x4 a[2][BM * 8];
  u32x4 b[2][BN * 8];
};

// XCD-aware remap: hardware deals workgroup ids round-robin over the 8 XCDs;
// give each XCD a contiguous range of logical ids (each XCD has its own L2).
__device__ __forceinline__ int xcd_lid(int bid, int nblk) {
  const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7, idx = bid >> 3;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}
// logical id -> (split, tile row, tile column), tiles grouped group_m rows deep
__device__ __forceinline__ void tile_of(const GemmDesc &d, int lid, int &tm, int &tn, int &split) {
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
__device__ __forceinline__ void tile_coords(const GemmDesc &d, int &tm, int &tn, int &split) {
  tile_of(d, xcd_lid(blockIdx.x, gridDim.x), tm, tn, split);
}

template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool VEC, bool KSEG>
__global__ void __launch_bounds__(NTHREADS) gemm_bf16_kernel(GemmDesc d) {
  __shared__ Smem<BM, BN> sm;
  constexpr bool DUAL = EPI == EPI_SWIGLU_FWD;
  static_assert(!(DUAL && (B_KC || KSEG)), "the dual gate/up operand is an n-contiguous weight");
  constexpr int WTM = BM / 2, WTN = BN / 2, FM = WTM / 32, FN = WTN / 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  int tm, tn, split;
  tile_coords(d, tm, tn, split);

  int sn = 0;  // N-segment of this tile
  if constexpr (!KSEG)
    while (sn + 1 < d.nseg && tn >= d.seg_tile0[sn + 1]) ++sn;
  constexpr int NCOLS = DUAL ? BN / 2 : BN;  // output columns per tile
  const int n0 = KSEG ? tn * BN : (tn - d.seg_tile0[sn]) * NCOLS;
  const int nlen = KSEG ? d.N : d.seg_len[sn];
  const int m0 = tm * BM;

  const int kt_total = KSEG ? d.seg_tile0[d.nseg] : (d.K + BK - 1) / BK;
  const int kt_begin = split * d.kt_per_split;
  const int kt_end = min(kt_total, kt_begin + d.kt_per_split);

  using LA = std::conditional_t<A_KC, LoadKC<BM, VEC>, LoadRC<BM, VEC, false>>;
  using LB = std::conditional_t<B_KC, LoadKC<BN, VEC>, LoadRC<BN, VEC, DUAL>>;
  LA la;
  LB lb;

  // K cursor: segment ks, offset k0 inside it (segments only with KSEG)
  int ks = 0, k0;
  if constexpr (KSEG) {
    while (ks + 1 < d.nseg && kt_begin >= d.seg_tile0[ks + 1]) ++ks;
    k0 = (kt_begin - d.seg_tile0[ks]) * BK;
  } else {
    k0 = kt_begin * BK;
  }
  // the upper half of the workgroup (waves 2, 3) loads the up weight in DUAL mode
  const int hi = __builtin_amdgcn_readfirstlane(tid >> 7);
  const uint16_t *Ab, *Bb;
  int64_t lda, ldb;
  int klen;
  auto set_seg = [&]() {
    const int ia = KSEG ? ks : 0, ib = KSEG ? ks : sn;
    Ab = (const uint16_t *)d.A[ia];
    lda = d.lda[ia];
    Bb = (const uint16_t *)(DUAL ? d.B[hi] : d.B[ib]);
    ldb = d.ldb[ib];
    klen = KSEG ? d.seg_len[ks] : d.K;
    la.init(lda, d.M - m0, tid);
    lb.init(ldb, nlen - n0, tid);
  };
  auto fetch = [&]() {
    const uint16_t *ta = A_KC ? Ab + (int64_t)m0 * lda + k0 : Ab + (int64_t)k0 * lda + m0;
    const uint16_t *tb = B_KC ? Bb + (int64_t)n0 * ldb + k0 : Bb + (int64_t)k0 * ldb + n0;
    la.load(ta, klen - k0, tid);
    lb.load(tb, klen - k0, tid);
  };
  auto advance = [&]() {  // only called when another K tile follows
    k0 += BK;
    if constexpr (KSEG) {
      if (k0 >= klen) {
        k0 = 0;
        ++ks;
        while (ks + 1 < d.nseg && d.seg_len[ks] == 0) ++ks;
        set_seg();
      }
    }
  };
  set_seg();

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // LDS row of the wave's fn-th 32-wide B fragment
  auto brow = [&](int fn) -> int {
    if constexpr (DUAL)
      return (fn < FN / 2) ? wn * (BN / 4) + fn * 32 : BN / 2 + wn * (BN / 4) + (fn - FN / 2) * 32;
    return wn * WTN + fn * 32;
  };

  if (kt_begin < kt_end) {
    fetch();
    la.store(sm.a[0], tid);
    lb.store(sm.b[0], tid);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) {
      advance();
      fetch();
    }
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

  float *ep = (float *)&sm + wid * 32 * (WTN + 8);
  // CE statistics: the per-row merge buffer sits after the 4 waves' strips
  static_assert(EPI != EPI_CE_STATS || 4 * (4 * 32 * (WTN + 8) + 4 * BM) <= (int)sizeof(sm), "CE buffer");
  epilogue<BM, BN, EPI, OUT_F32, VEC, DUAL>(d, acc, ep, lane, wm, wn, m0, n0, nlen, KSEG ? 0 : sn, split,
                                            (float *)&sm + 4 * 32 * (WTN + 8));
}

// ===========================================================================
// Main kernel: operands move global -> LDS by buffer DMA (no register staging)
// ===========================================================================
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) char lds_char_t;

// k-contiguous tiles [rows][64 k]: 16-byte chunk c of row r sits at c ^ swk(r).
// Eight consecutive rows hit eight different chunks (conflict-free fragment
// reads), and the pattern repeats every 32 rows, so fragments 32 rows apart
// are a fixed byte offset from each other.
__device__ __forceinline__ int swk(int r) { return (r & 7) ^ ((r >> 3) & 3); }
// row-contiguous tiles [64 k][C*8]: chunk c of k-row k sits at c ^ swr(k); the
// 4 k-rows x 32 columns read by half a wave's transpose loads land on 16
// distinct 16-byte bank groups.  With 24 chunks (192 columns, 384-byte k-rows,
// which alternate between the two 128-byte halves of the bank array) flipping
// chunk bit 2 on every other pair of k-rows is enough, and it keeps c < 24.
template <int C>
__device__ __forceinline__ int swr(int k) { return (C == 16 || C == 32) ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

// buffer resource words for a wave-uniform base pointer
__device__ __forceinline__ i32x4 rsrc_words(const void *p) {
  const uint64_t b = (uint64_t)p;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
  r[2] = NREC;
  r[3] = RSRC_W3;
  return r;
}
// 16 bytes per lane from buffer offset voff + soff straight into LDS at
// lds + 16 * lane.  Issued as asm so that the compiler does not treat the
// in-flight DMA as an LDS store every later LDS read must wait for (it would
// wait for the next tile too); the kernel waits on vmcnt explicitly before the
// barrier that publishes a tile.  The memory clobber keeps LDS accesses in order.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_char_t *)p;
}
// workgroup barrier without the memory fence of __syncthreads(): the fence
// would make every wave drain all of its DMA, including the next tile's
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One operand tile (R rows of 64 k, or 64 k-rows of R columns) staged by
// R/(8 NW) one-kilobyte DMA instructions per wave (NW waves).  DUAL: the R columns are two
// sub-tiles of R/2 from two matrices; the first half of the waves fills the first, the
// second half the second.
template <int R, bool KC, bool DUAL, int NW = 4>
struct Dma {
  static constexpr int NI = R / (8 * NW);  // kilobytes per wave
  static constexpr int REFF = DUAL ? R / 2 : R;   // columns of one row-contiguous sub-tile
  static constexpr int P = 2 * REFF;              // its k-row pitch (bytes)
  uint32_t vo[NI];   // per-lane byte offset within the block
  uint32_t so[NI];   // wave-uniform byte offset of the block's first row / k-row
  int extent;        // rows (KC) or columns (RC) from the tile origin to the matrix edge
  __device__ __forceinline__ int blk(int wave, int i) const {
    const int b = wave * NI + i;
    return (!KC && DUAL) ? b % (REFF / 8) : b;
  }
  __device__ __forceinline__ void init(int64_t ld, int extent_, int wave, int lane) {
    extent = extent_;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int bl = blk(wave, i);
      if constexpr (KC) {
        so[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(bl * 8 * ld * 2));
        const int r = 8 * bl + (lane >> 3);
        const int c = (lane & 7) ^ swk(r);
        vo[i] = (uint32_t)((lane >> 3) * ld * 2 + c * 16);
      } else {
        // the kilobyte may start inside a k-row (P = 384)
        const int q = bl * 1024 + lane * 16, kf = bl * 1024 / P;
        const int k = q / P;
        const int c = (q % P / 16) ^ swr<REFF / 8>(k);
        so[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(kf * ld * 2));
        vo[i] = (uint32_t)((k - kf) * ld * 2 + c * 16);
      }
    }
  }
  // lane offsets for one K tile (masked on tiles that cross the K or row/column edge)
  __device__ __forceinline__ void offsets(uint32_t *o, int kleft, int wave, int lane) const {
    const bool edge = kleft < BK || extent < (KC ? R : REFF);
#pragma unroll
    for (int i = 0; i < NI; ++i) o[i] = vo[i];
    if (edge) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int bl = blk(wave, i);
        if constexpr (KC) {
          const int r = 8 * bl + (lane >> 3);
          const int c = (lane & 7) ^ swk(r);
          if (r >= extent || c * 8 >= kleft) o[i] = OOB;
        } else {
          const int q = bl * 1024 + lane * 16;
          const int k = q / P;
          const int c = (q % P / 16) ^ swr<REFF / 8>(k);
          if (k >= kleft || c * 8 >= extent) o[i] = OOB;
        }
      }
    }
  }
  __device__ __forceinline__ void issue(const i32x4 &rs, const uint32_t *o, int i, uint32_t region,
                                        int wave) const {
    dma16(rs, o[i], so[i], region + (wave * NI + i) * 1024);
  }
};

// byte offset (stage-relative) of the first of the two 8-byte transpose reads
// that give lane l the 4+4 k values of column col0 + l%32 of a row-contiguous
// sub-tile with pitch P and C chunks per row (h selects the second read)
__device__ __forceinline__ int rc_frag_off(int P, int C, int col0, int h, int lane) {
  const int g = (lane >> 4) & 3, j = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  const int k = 8 * (g >> 1) + (j >> 2) + 4 * h;
  const int sw = (C == 16 || C == 32) ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
  return k * P + (((col >> 3) ^ sw) << 4) + ((col & 7) << 1);
}
__device__ __forceinline__ bf16x8 read_tr(const char *p0, const char *p1) {
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)p0);
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)p1);
  const short8v v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The whole tile computation of the DMA kernel for logical tile id `lid`;
// smem0 / smem1 are the two LDS stages (each at least 128 * (BM + BN) bytes)
// declared by the calling kernel.
template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool KSEG, int NW = 4, int NS = 2,
          bool A3 = false>
__device__ __forceinline__ void dma_body(const GemmDesc &d, int lid, char *smem0, char *smem1,
                                         char *smem2 = nullptr) {
  static_assert(NS == 2 || NS == 3, "two or three LDS stages");
  constexpr bool DUAL = EPI == EPI_SWIGLU_FWD;
  static_assert(!(DUAL && (B_KC || KSEG)), "the dual gate/up operand is an n-contiguous weight");
  static_assert(!A3 || (NS == 2 && !KSEG && !DUAL), "three A stages: two-stage single-B products");
  // NW waves in a 2 x NW/2 grid, each a (BM/2) x (BN/(NW/2)) sub-tile
  constexpr int WGN = NW / 2;
  constexpr int WTM = BM / 2, WTN = BN / WGN, FM = WTM / 32, FN = WTN / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WGN, wn = wid % WGN;

  int tm, tn, split;
  tile_of(d, lid, tm, tn, split);
  int sn = 0;  // N-segment of this tile
  if constexpr (!KSEG)
    while (sn + 1 < d.nseg && tn >= d.seg_tile0[sn + 1]) ++sn;
  constexpr int NCOLS = DUAL ? BN / 2 : BN;
  const int n0 = KSEG ? tn * BN : (tn - d.seg_tile0[sn]) * NCOLS;
  const int nlen = KSEG ? d.N : d.seg_len[sn];
  const int m0 = tm * BM;
  const int kt_total = KSEG ? d.seg_tile0[d.nseg] : (d.K + BK - 1) / BK;
  const int kt_begin = split * d.kt_per_split;
  const int kt_end = min(kt_total, kt_begin + d.kt_per_split);

  using DA = Dma<BM, A_KC, false, NW>;
  using DB = Dma<BN, B_KC, DUAL, NW>;
  constexpr int NLD = DA::NI + DB::NI;  // DMA instructions per wave per tile
  DA da;
  DB db;

  // K cursor over the segments: the next tile to stage is (ks, k0)
  int ks = 0, k0;
  if constexpr (KSEG) {
    while (ks + 1 < d.nseg && kt_begin >= d.seg_tile0[ks + 1]) ++ks;
    k0 = (kt_begin - d.seg_tile0[ks]) * BK;
  } else {
    k0 = kt_begin * BK;
  }
  const uint16_t *Ab, *Bb;
  int64_t lda, ldb;
  int klen;
  auto set_seg = [&]() {
    const int ia = KSEG ? ks : 0, ib = KSEG ? ks : sn;
    Ab = (const uint16_t *)d.A[ia];
    lda = d.lda[ia];
    Bb = (const uint16_t *)(DUAL ? d.B[wid / (NW / 2)] : d.B[ib]);
    ldb = d.ldb[ib];
    klen = KSEG ? d.seg_len[ks] : d.K;
    da.init(lda, d.M - m0, wid, lane);
    db.init(ldb, nlen - n0, wid, lane);
  };
  set_seg();
  i32x4 rsa, rsb;
  uint32_t oa[DA::NI], ob[DB::NI];
  // descriptors and lane offsets of the tile at the cursor; then advance it
  auto prep = [&]() {
    if constexpr (KSEG) {
      if (k0 >= klen) {
        k0 = 0;
        ++ks;
        while (ks + 1 < d.nseg && d.seg_len[ks] == 0) ++ks;
        set_seg();
      }
    }
    const uint16_t *ta = A_KC ? Ab + (int64_t)m0 * lda + k0 : Ab + (int64_t)k0 * lda + m0;
    const uint16_t *tb = B_KC ? Bb + (int64_t)n0 * ldb + k0 : Bb + (int64_t)k0 * ldb + n0;
    rsa = rsrc_words(ta);
    rsb = rsrc_words(tb);
    da.offsets(oa, klen - k0, wid, lane);
    db.offsets(ob, klen - k0, wid, lane);
    k0 += BK;
  };
  auto dma_q = [&](int q, uint32_t stage) {
    if (q < DA::NI) da.issue(rsa, oa, q, stage, wid);
    else db.issue(rsb, ob, q - DA::NI, stage + 128 * BM, wid);
  };

  // per-lane fragment byte offsets (stage-relative)
  int aoff[4], boff[4], arc[FM][2], brc[FN][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ra = wm * WTM + (lane & 31);
    aoff[kk] = ra * 128 + (((kk * 2 + (lane >> 5)) ^ swk(ra)) << 4);
    const int rb = wn * WTN + (lane & 31);
    boff[kk] = 128 * BM + rb * 128 + (((kk * 2 + (lane >> 5)) ^ swk(rb)) << 4);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int h = 0; h < 2; ++h) arc[fm][h] = rc_frag_off(2 * BM, BM / 8, wm * WTM + fm * 32, h, lane);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (DUAL)
        brc[fn][h] = 128 * BM + (fn < FN / 2 ? 0 : 64 * BN) +
                     rc_frag_off(BN, BN / 16, wn * (BN / NW) + (fn % (FN / 2)) * 32, h, lane);
      else
        brc[fn][h] = 128 * BM + rc_frag_off(2 * BN, BN / 8, wn * WTN + fn * 32, h, lane);
    }
  auto load_frags = [&](const char *S, int kk, bf16x8 *af, bf16x8 *bfr) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if constexpr (A_KC) af[fm] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + aoff[kk] + fm * 32 * 128));
      else af[fm] = read_tr(S + arc[fm][0] + kk * 16 * 2 * BM, S + arc[fm][1] + kk * 16 * 2 * BM);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      if constexpr (B_KC) {
        bfr[fn] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + boff[kk] + fn * 32 * 128));
      } else {
        constexpr int PB = DUAL ? BN : 2 * BN;
        bfr[fn] = read_tr(S + brc[fn][0] + kk * 16 * PB, S + brc[fn][1] + kk * 16 * PB);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // One K step on stage S.  The fragments of 16-deep slice kk+1 are read before
  // the MFMAs of slice kk, and the next tile's DMAs are spread between the MFMA
  // groups of slices 0 and 1; sched_barrier fences pin both orders.  The single
  // barrier per step (before it) retired the stage these DMAs overwrite.
  constexpr int GROUPS = 2 * FM;
  constexpr int PER = (NLD + GROUPS - 1) / GROUPS;
  auto step = [&](const char *__restrict__ S, uint32_t nxt, bool more) {
    bf16x8 fa[2][FM], fb[2][FN];
    load_frags(S, 0, fa[0], fb[0]);
    if (more) prep();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) load_frags(S, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][fm], fb[kk & 1][fn], acc[fm][fn], 0, 0, 0);
        if (kk < 2 && more) {
          const int g = kk * FM + fm;
#pragma unroll
          for (int p = 0; p < PER; ++p)
            if (g * PER + p < NLD) dma_q(g * PER + p, nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const uint32_t L0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem0));
  const uint32_t L1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem1));
  const int nk = kt_end - kt_begin;
  if constexpr (A3) {
    // Three A stages and two B stages in [A0 | A1 | A2 | B0 | B1]: step t stages B of
    // tile t+1 and then A of tile t+2 (each into the buffer step t-1 used), so an A
    // tile has two steps to land.  The waves' DMAs retire in issue order, so waiting
    // until at most A(t+1)'s are outstanding means A(t) and B(t) have landed.
    char *const abase = smem0, *const bbase = smem0 + 3 * 128 * BM;
    const uint32_t LA = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(abase));
    const uint32_t LB = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(bbase));
    int kA = k0, kB = k0;
    auto prepA = [&]() {
      rsa = rsrc_words(A_KC ? Ab + (int64_t)m0 * lda + kA : Ab + (int64_t)kA * lda + m0);
      da.offsets(oa, klen - kA, wid, lane);
      kA += BK;
    };
    auto prepB = [&]() {
      rsb = rsrc_words(B_KC ? Bb + (int64_t)n0 * ldb + kB : Bb + (int64_t)kB * ldb + n0);
      db.offsets(ob, klen - kB, wid, lane);
      kB += BK;
    };
    // A's fragments from SA, B's from SB (B offsets carry the 128 * BM of a whole stage)
    auto load_frags2 = [&](const char *SA, const char *SB, int kk, bf16x8 *af, bf16x8 *bfr) {
      const char *SBv = SB - 128 * BM;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if constexpr (A_KC) af[fm] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(SA + aoff[kk] + fm * 32 * 128));
        else af[fm] = read_tr(SA + arc[fm][0] + kk * 16 * 2 * BM, SA + arc[fm][1] + kk * 16 * 2 * BM);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if constexpr (B_KC) bfr[fn] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(SBv + boff[kk] + fn * 32 * 128));
        else bfr[fn] = read_tr(SBv + brc[fn][0] + kk * 16 * 2 * BN, SBv + brc[fn][1] + kk * 16 * 2 * BN);
      }
    };
    if (nk > 0) {
      prepA();
#pragma unroll
      for (int i = 0; i < DA::NI; ++i) da.issue(rsa, oa, i, LA, wid);
      prepB();
#pragma unroll
      for (int i = 0; i < DB::NI; ++i) db.issue(rsb, ob, i, LB, wid);
    }
    if (nk > 1) {
      prepA();
#pragma unroll
      for (int i = 0; i < DA::NI; ++i) da.issue(rsa, oa, i, LA + 128 * BM, wid);
    }
    int sa = 0;  // A stage of tile t
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DA::NI) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      const char *SA = abase + sa * 128 * BM, *SB = bbase + (t & 1) * 128 * BN;
      const bool moreB = t + 1 < nk, moreA = t + 2 < nk;
      const uint32_t nB = LB + ((t + 1) & 1) * 128 * BN;
      const uint32_t nA = LA + (sa == 0 ? 2 : sa - 1) * 128 * BM;  // stage (t + 2) % 3
      bf16x8 fa[2][FM], fb[2][FN];
      load_frags2(SA, SB, 0, fa[0], fb[0]);
      if (moreB) prepB();
      if (moreA) prepA();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) load_frags2(SA, SB, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][fm], fb[kk & 1][fn], acc[fm][fn], 0, 0, 0);
          if (kk < 2) {
            const int g = kk * FM + fm;
#pragma unroll
            for (int p = 0; p < PER; ++p) {
              const int q = g * PER + p;  // B's DMAs first, then A's
              if (q < DB::NI) {
                if (moreB) db.issue(rsb, ob, q, nB, wid);
              } else if (q < NLD) {
                if (moreA) da.issue(rsa, oa, q - DB::NI, nA, wid);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      sa = sa == 2 ? 0 : sa + 1;
    }
  } else if constexpr (NS == 2) {
    if (nk > 0) {
      prep();
#pragma unroll
      for (int q = 0; q < NLD; ++q) dma_q(q, L0);
    }
    for (int t = 0; t < nk; ++t) {
      const char *cur = (t & 1) ? smem1 : smem0;
      const uint32_t nxt = (t & 1) ? L0 : L1;
      // this wave's DMA of tile t is the only DMA outstanding here
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      step(cur, nxt, t + 1 < nk);
    }
  } else {
    // three stages: tile t+2 is staged while tile t is multiplied, so a DMA has
    // two steps to land
    const uint32_t L2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem2));
    if (nk > 0) {
      prep();
#pragma unroll
      for (int q = 0; q < NLD; ++q) dma_q(q, L0);
    }
    if (nk > 1) {
      prep();
#pragma unroll
      for (int q = 0; q < NLD; ++q) dma_q(q, L1);
    }
    int sc = 0;  // stage of tile t
    for (int t = 0; t < nk; ++t) {
      const char *cur = sc == 0 ? smem0 : (sc == 1 ? smem1 : smem2);
      const uint32_t nxt = sc == 0 ? L2 : (sc == 1 ? L0 : L1);
      // the wave's DMAs retire in issue order: at most tile t+1's may stay outstanding
      if (t + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      step(cur, nxt, t + 2 < nk);
      sc = sc == 2 ? 0 : sc + 1;
    }
  }

  // epilogue strips: the first half of the waves in stage 0, the rest in stage 1 (the first
  // __syncthreads inside the epilogue retires the last tile)
  float *ep = (float *)(wid < NW / 2 ? smem0 : smem1) + (wid % (NW / 2)) * 32 * (WTN + 8);
  if constexpr ((EPI == EPI_STORE && OUT_F32) || EPI == EPI_PARTIAL) {
    epilogue_f32_direct<BM, BN, NW, EPI == EPI_PARTIAL>(d, acc, lane, wm, wn, m0, n0, nlen, KSEG ? 0 : sn, split);
    return;
  }
  // CE statistics: the per-row merge buffer sits in stage 0 after the first half's strips
  static_assert(EPI != EPI_CE_STATS || 4 * ((NW / 2) * 32 * (WTN + 8) + NW * BM) <= 128 * (BM + BN), "CE buffer");
  epilogue<BM, BN, EPI, OUT_F32, true, DUAL, NW>(d, acc, ep, lane, wm, wn, m0, n0, nlen, KSEG ? 0 : sn, split,
                                                 (float *)smem0 + (NW / 2) * 32 * (WTN + 8));
}

// Sum the split-K partials in split order (deterministic) and store.  Each
// thread owns a run of 8 columns of one row (VEC: N and the segment widths
// are multiples of 8); the scalar build owns single elements.
template <bool OUT_F32, bool VEC>
__device__ __forceinline__ void splitk_reduce_body(const GemmDesc &d, int64_t first, int64_t stride) {
  constexpr int W = VEC ? 8 : 1;
  const int runs = d.N / W;
  const int64_t total = (int64_t)d.M * runs;
  for (int64_t i = first; i < total; i += stride) {
    const int gm = (int)(i / runs);
    const int gc = (int)(i - (int64_t)gm * runs) * W;
    float s[W];
#pragma unroll
    for (int q = 0; q < W; ++q) s[q] = 0.f;
    // up to 8 splits' loads in flight before their sums (in split order)
    for (int k0 = 0; k0 < d.splits; k0 += 8) {
      float4 a[8], b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < d.splits) {
          const float *p = d.ws + ((int64_t)(k0 + j) * d.M + gm) * d.N + gc;
          if constexpr (VEC) {
            a[j] = *(const float4 *)p;
            b[j] = *(const float4 *)(p + 4);
          } else {
            a[j].x = p[0];
          }
        }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < d.splits) {
          if constexpr (VEC) {
            s[0] += a[j].x; s[1] += a[j].y; s[2] += a[j].z; s[3] += a[j].w;
            s[4] += b[j].x; s[5] += b[j].y; s[6] += b[j].z; s[7] += b[j].w;
          } else {
            s[0] += a[j].x;
          }
        }
    }
    int sg = 0;
    if (!d.kseg)
      while (sg + 1 < d.nseg && gc >= d.seg_col0[sg + 1]) ++sg;
    const int cc = d.kseg ? gc : gc - d.seg_col0[sg];
    const int si = d.kseg ? 0 : sg;
    if constexpr (OUT_F32) {
      float *o = (float *)d.C[si] + (int64_t)gm * d.ldc[si] + cc;
      if constexpr (VEC) {
        *(float4 *)o = make_float4(s[0], s[1], s[2], s[3]);
        *(float4 *)(o + 4) = make_float4(s[4], s[5], s[6], s[7]);
      } else {
        o[0] = s[0];
      }
    } else {
      uint16_t *o = (uint16_t *)d.C[si] + (int64_t)gm * d.ldc[si] + cc;
      if constexpr (VEC) *(u32x4 *)o = pack8(s);
      else o[0] = tp_f2bf(s[0]);
    }
  }
}

template <bool OUT_F32, bool VEC>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmDesc d) {
  splitk_reduce_body<OUT_F32, VEC>(d, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                                   (int64_t)gridDim.x * blockDim.x);
}

}  // namespace

template <int BM_, int BN_, bool A_KC_, bool B_KC_, int EPI_, bool OUT_F32_, bool KSEG_>
struct Cfg {
  static constexpr int STAGE = 128 * (BM_ + BN_);
  // LDS of three A stages and two B stages (the A-deep pipeline of single-B products)
  static constexpr int A3_LDS = 128 * (3 * BM_ + 2 * BN_);
  static constexpr bool A3_OK = !KSEG_ && EPI_ != EPI_SWIGLU_FWD;
  template <int NS, int NW, bool A3 = false>
  static __device__ __forceinline__ void run(const GemmDesc &d, int lid, char *s0, char *s1, char *s2) {
    dma_body<BM_, BN_, A_KC_, B_KC_, EPI_, OUT_F32_, KSEG_, NW, NS, A3>(d, lid, s0, s1, s2);
  }
};

// waves per SIMD of a residency (4 SIMDs per CU)
constexpr int res_wpe(int res) { return res_wgs(res) * res_waves(res) / 4; }

template <int BM, int BN, bool A_KC, bool B_KC, int EPI, bool OUT_F32, bool KSEG, int RES>
__global__ void __launch_bounds__(64 * res_waves(RES))
__attribute__((amdgpu_waves_per_eu(res_wpe(RES), res_wpe(RES)))) gemm_dma_kernel(GemmDesc d) {
  static_assert(res_fits(BM, BN, RES), "LDS stages exceed the CU's 160 KB");
  constexpr int S = 128 * (BM + BN), NS = res_stages(RES);
  // one 8-wave workgroup per CU: the LDS left over by two stages takes a third A stage
  constexpr bool A3 = RES == RES_WAVES8 && !KSEG && EPI != EPI_SWIGLU_FWD && 128 * (3 * BM + 2 * BN) <= 160 * 1024;
  constexpr int LDS = A3 ? 128 * (3 * BM + 2 * BN) : NS * S;
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  dma_body<BM, BN, A_KC, B_KC, EPI, OUT_F32, KSEG, res_waves(RES), NS, A3>(
      d, xcd_lid(blockIdx.x, gridDim.x), smem, smem + S, NS == 3 ? smem + 2 * S : nullptr);
}

// Two independent products in one launch: workgroups [0, n1) compute the
// first, [n1, n1 + n2) the second.  The first is the one with the longer tiles
// (a long-K weight gradient), so its workgroups are dispatched first and the
// short tiles of the second fill the CUs around them.  Each range gets the XCD
// remap when n1 is a multiple of 8 (then both ranges start on XCD 0).  The last
// n3 workgroups sum the split-K partials of an earlier launch's product (d3,
// bf16 output, 16-byte runs): they are dispatched as the tiles drain.
template <class C1, class C2, int RES>
__global__ void __launch_bounds__(64 * res_waves(RES))
__attribute__((amdgpu_waves_per_eu(res_wpe(RES), res_wpe(RES)))) gemm_dma_pair_kernel(GemmDesc d1, GemmDesc d2,
                                                                                      int n1, int n2,
                                                                                      GemmDesc d3, int n3) {
  constexpr int S = C1::STAGE > C2::STAGE ? C1::STAGE : C2::STAGE, NS = res_stages(RES);
  static_assert(NS * res_wgs(RES) * S <= 160 * 1024, "LDS stages exceed the CU's 160 KB");
  // with one 8-wave workgroup per CU, a product that can takes a third A stage
  constexpr bool A3_1 = RES == RES_WAVES8 && C1::A3_OK && C1::A3_LDS <= 160 * 1024;
  constexpr bool A3_2 = RES == RES_WAVES8 && C2::A3_OK && C2::A3_LDS <= 160 * 1024;
  constexpr int L1 = A3_1 ? C1::A3_LDS : NS * S, L2 = A3_2 ? C2::A3_LDS : NS * S;
  __shared__ __attribute__((aligned(1024))) char smem[L1 > L2 ? L1 : L2];
  char *s2 = NS == 3 ? smem + 2 * S : nullptr;
  const int b = blockIdx.x;
  if (b >= n1 + n2) {
    const int64_t nt = 64 * res_waves(RES);
    splitk_reduce_body<false, true>(d3, (int64_t)(b - n1 - n2) * nt + threadIdx.x, (int64_t)n3 * nt);
    return;
  }
  const bool remap = (n1 & 7) == 0;
  if (b < n1) {
    C1::template run<NS, res_waves(RES), A3_1>(d1, remap ? xcd_lid(b, n1) : b, smem, smem + S, s2);
  } else {
    const int r = b - n1;
    C2::template run<NS, res_waves(RES), A3_2>(d2, remap ? xcd_lid(r, n2) : r, smem, smem + S, s2);
  }
}

