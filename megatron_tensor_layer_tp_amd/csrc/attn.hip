// attn.hip -- attention core on a shard's heads: causal scaled dot-product
// attention of the nq query heads a tensor-parallel shard holds, sharing its nkv
// key/value heads ("7.3 模型并行与张量并行" §7.3.4: each card runs attention on
// its own 8 of the 64 query heads and 1 of the 8 KV heads, then concatenates
// them to [s, 1024]).  Flash-style (the CS336 lecture-8 book's activation-memory
// section: FlashAttention never stores the s x s scores): scores live in
// registers one 64-key tile at a time, with a running max and sum per query.
//
// Design (CDNA4, head dim 128):
//  * A workgroup of 8 wave64s (two per SIMD, <= 256 VGPRs each, so one wave's
//    softmax arithmetic overlaps the other's MFMAs) works on one head.  Its two
//    4-wave groups take the same 128 query rows (32 per wave) and split the key
//    tiles in halves, then merge their running max, sum and O through LDS.
//  * Both products run transposed, S^T = K . Q^T and O^T = V^T . P^T, with
//    v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane then
//    holds a single query column, so the running max, the sum and the rescale
//    of O are per-lane scalars, and P^T feeds the second product straight from
//    the first one's registers (its keys come in a lane-local order that the
//    V^T fragments, read with the LDS transpose read, follow).
//  * K and V tiles [64 keys][128 d] are staged by buffer DMA into two LDS stages
//    (the next tile's DMA runs during the current tile's math).  K chunks are
//    XOR-swizzled by the row (conflict-free 16-byte fragment reads), V chunks by
//    4 (row & 3) (conflict-free transpose reads).
//  * Causal: a block reads keys 0 .. its last query; a wave skips the tiles past
//    its last query and masks only the tiles that cross its diagonal.  Each
//    workgroup takes query blocks i and nqb-1-i one after the other, so every
//    workgroup has the same number of key tiles.
//  * Output: O rows in bf16 through an LDS transpose (16-byte stores), and the
//    natural log-sum-exp of each row's scores in fp32.
#include "gemm_bf16_kernels.h"

namespace {

constexpr int HD = 128;                  // head dimension
constexpr int QB = 128;                  // query rows per workgroup
constexpr int KT = 64;                   // keys per tile
constexpr int TILE = KT * HD * 2;        // bytes of one K or V tile

struct AttnArgs {
  const uint16_t *Q, *K, *V;
  uint16_t *O;
  float *lse;
  int s, nq, nkv, nqb;
  int64_t ldq, ldk;  // elements per row of Q and O, of K and V
  float c;           // log2(e) / sqrt(d)
  float rescale;     // 8 / c: the raw-score headroom over the reference max
};

// K tile: 16-byte chunk c of key row r sits at c ^ (r & 15)
__device__ __forceinline__ int koff(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
// V tile: chunk of column col in key row r sits at (col / 8) ^ 4 (r & 3)
__device__ __forceinline__ int voff(int r, int col) {
  return r * 256 + ((((col >> 3) ^ (4 * (r & 3)))) << 4) + ((col & 7) << 1);
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(AttnArgs a) {
  // [group][stage][K tile | V tile]
  __shared__ __attribute__((aligned(1024))) char sm[2][2][2 * TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wl = w & 3;
  const int h = lane >> 5, ql = lane & 31;
  const int head = blockIdx.x % a.nq;
  const int pair = blockIdx.x / a.nq;
  const int g = head / (a.nq / a.nkv);
  char *const mine = sm[grp][0];
  char *const merge_o = sm[1][0];          // group 1's O partials: [4 waves][64 values][64 lanes] fp32
  float *const merge_ml = (float *)sm[0][0];  // group 1's m and l: [4 waves][2][64 lanes]

  // DMA: in each group, wave wl stages kilobytes 4wl .. 4wl+3 of the K and the V tile
  uint32_t kvo[4], vvo[4];
  int krow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * wl + i, r = 4 * b + (lane >> 4), pos = lane & 15;
    krow[i] = r;
    kvo[i] = (uint32_t)(r * a.ldk * 2 + ((pos ^ (r & 15)) << 4));
    vvo[i] = (uint32_t)(r * a.ldk * 2 + ((pos ^ (4 * (r & 3))) << 4));
  }
  const uint32_t L0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sm[grp][0]));
  const uint32_t L1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sm[grp][1]));
  auto issue = [&](int t, uint32_t stage) {
    const int k0 = t * KT;
    const i32x4 rk = rsrc_words(a.K + (int64_t)k0 * a.ldk + g * HD);
    const i32x4 rv = rsrc_words(a.V + (int64_t)k0 * a.ldk + g * HD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = k0 + krow[i] < a.s;
      dma16(rk, in ? kvo[i] : OOB, 0u, stage + (4 * wl + i) * 1024);
      dma16(rv, in ? vvo[i] : OOB, 0u, stage + TILE + (4 * wl + i) * 1024);
    }
  };

  // per-lane fragment offsets (stage-relative)
  int ko[2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 8; ++t) ko[kb][t] = koff(32 * kb + ql, 2 * t + h);
  // V^T fragment of (d block db, key slice t): two transpose reads of 4 key rows,
  // rows 16t + 4h + (0..3) and 16t + 8 + 4h + (0..3) -- the order the keys of P^T
  // have in this lane's accumulator -- at column 32 db + 16 ((lane >> 4) & 1) + 4 (j & 3)
  int vo[4][2];
  {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      vo[db][0] = TILE + voff(4 * h + (j >> 2), col);
      vo[db][1] = TILE + voff(8 + 4 * h + (j >> 2), col);
    }
  }

  // Causal balance: the workgroup takes query blocks `pair` and nqb-1-pair (equal
  // total length), and for each block its two 4-wave groups split the key tiles
  // in halves -- group 0 the first, group 1 the second (with the diagonal) --
  // then merge (max, sum, O) through LDS.
  const int blocks[2] = {a.nqb - 1 - pair, pair};
  const int nblk = blocks[0] == blocks[1] ? 1 : 2;
  for (int bi = 0; bi < nblk; ++bi) {
    const int q0 = blocks[bi] * QB, qw0 = q0 + 32 * wl, myq = qw0 + ql;
    bf16x8 qf[8];  // Q^T fragments: slice t holds d = 16t + 8h .. 16t + 8h + 7
    {
      const uint16_t *qp = a.Q + (int64_t)min(myq, a.s - 1) * a.ldq + head * HD + 8 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 v = myq < a.s ? *(const u32x4 *)(qp + 16 * t) : zero4();
        qf[t] = __builtin_bit_cast(bf16x8, v);
      }
    }
    const int kend = min(q0 + QB, a.s);  // keys the block needs: 0 .. kend - 1
    const int n = (kend + KT - 1) / KT;
    const int n0 = n / 2;
    const int tbeg = grp ? n0 : 0, tcnt = grp ? n - n0 : n0;
    const int iters = n - n0;               // >= n0: both groups pass the same barriers
    const int wkend = min(qw0 + 32, a.s);   // keys this wave needs
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    if (tcnt > 0) issue(tbeg, L0);
    for (int it = 0; it < iters; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (it + 1 < tcnt) issue(tbeg + it + 1, (it & 1) ? L0 : L1);
      const int k0 = (tbeg + it) * KT;
      if (it >= tcnt || k0 >= wkend) continue;  // wave-uniform
      const char *S = mine + (it & 1) * 2 * TILE;

      // S^T = K . Q^T for keys k0 .. k0+63 (two 32-key blocks)
      f32x16 sa[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[kb][e] = 0.f;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + ko[kb][tt]));
          sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[tt], sa[kb], 0, 0, 0);
        }
      }

      // online softmax in base 2 on the raw scores (the scale c = log2(e)/sqrt(d)
      // is folded into the exponent's FMA); element e of block kb is key
      // k0 + 32 kb + 8 (e/4) + 4h + e%4.  Only tiles that cross the wave's
      // diagonal are masked.
      float mx = -INFINITY;
      if (k0 + KT - 1 > qw0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float v = sa[kb][e];
            if (k0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3) > myq) v = -INFINITY;
            sa[kb][e] = v;
            mx = fmaxf(mx, v);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sa[kb][e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // The reference max m moves only when a score exceeds it by more than
      // RESCALE (so exp2 arguments stay <= 8 and P <= 256): the rescale of the
      // sum and of O becomes rare once the running max has settled.
      float corr = 1.f;
      if (mx > m + a.rescale) {
        corr = tp_exp2((m - mx) * a.c);  // 0 on the first tile (m = -inf)
        m = mx;
      }
      const float mc = m * a.c;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = tp_exp2(fmaf(sa[kb][e], a.c, -mc));
          sa[kb][e] = p;
          ps += p;
        }
      l = fmaf(l, corr, ps);
      if (__any(corr != 1.f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= corr;
      }

      // O^T += V^T . P^T over four 16-key slices
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = sa[tt >> 1][8 * (tt & 1) + i];
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8(pv));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 vf = read_tr(S + vo[db][0] + tt * 16 * 256, S + vo[db][1] + tt * 16 * 256);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }

    // merge: group 1 hands (m, l, O) of each lane to the group-0 wave with the same queries
    __syncthreads();
    if (grp == 1) {
      float *po = (float *)merge_o + wl * 64 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) po[(16 * db + e) * 64] = o[db][e];
      merge_ml[(wl * 2) * 64 + lane] = m;
      merge_ml[(wl * 2 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = merge_ml[(wl * 2) * 64 + lane], l1 = merge_ml[(wl * 2 + 1) * 64 + lane];
      const float mt = fmaxf(m, m1);
      const float a0 = tp_exp2((m - mt) * a.c), a1 = tp_exp2((m1 - mt) * a.c);
      const float *po = (const float *)merge_o + wl * 64 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = o[db][e] * a0 + po[(16 * db + e) * 64] * a1;
      l = l * a0 + l1 * a1;
      m = mt;
      // the two lane halves hold disjoint keys of the same query
      const float lt = l + __shfl_xor(l, 32, 64);
      const float inv = 1.f / lt;
      if (h == 0 && myq < a.s) a.lse[(int64_t)head * a.s + myq] = (m * a.c + log2f(lt)) * 0.69314718055994531f;
      // O rows through LDS: this wave's [32 q][128 d] bf16, chunks XOR-swizzled by the row
      char *ob = sm[0][1] + wl * 8192;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = o[db][4 * j4 + i] * inv;
#pragma unroll
          for (int i = 4; i < 8; ++i) v[i] = 0.f;
          const u32x4 pk = pack8(v);
          uint2 two;
          two.x = pk[0];
          two.y = pk[1];
          *(uint2 *)(ob + ql * 256 + (((4 * db + j4) ^ (ql & 15)) << 4) + 8 * h) = two;
        }
      // the wave reads back only its own strip, and a wave's LDS operations
      // complete in order: no workgroup barrier (group 1 does not come here)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int idx = it * 64 + lane, r = idx >> 4, c = idx & 15;
        const u32x4 v = *(const u32x4 *)(ob + r * 256 + ((c ^ (r & 15)) << 4));
        if (qw0 + r < a.s) *(u32x4 *)(a.O + (int64_t)(qw0 + r) * a.ldq + head * HD + c * 8) = v;
      }
    }
    __syncthreads();  // LDS is reused by the next block
  }
}

}  // namespace

hipError_t tp_launch_attn_fwd(int64_t s, int64_t nq, int64_t nkv, const void *Q, const void *K, const void *V,
                              void *O, float *lse, hipStream_t st) {
  if (s == 0 || nq == 0) return hipSuccess;
  AttnArgs a;
  a.Q = (const uint16_t *)Q;
  a.K = (const uint16_t *)K;
  a.V = (const uint16_t *)V;
  a.O = (uint16_t *)O;
  a.lse = lse;
  a.s = (int)s;
  a.nq = (int)nq;
  a.nkv = (int)nkv;
  a.nqb = (int)((s + QB - 1) / QB);
  a.ldq = nq * HD;
  a.ldk = nkv * HD;
  a.c = 1.4426950408889634f / sqrtf((float)HD);
  a.rescale = 8.f / a.c;
  const int64_t pairs = (a.nqb + 1) / 2;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)(pairs * nq)), dim3(512), 0, st, a);
  return hipGetLastError();
}
