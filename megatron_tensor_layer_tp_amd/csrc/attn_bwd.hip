// attn_bwd.hip -- backward of the attention core on a shard's heads: dO -> dQ,
// dK, dV for the causal scaled dot-product attention of the nq query heads a
// tensor-parallel shard holds, sharing its nkv key/value heads ("7.3 模型并行与
// 张量并行" §7.3.4: each card runs attention on its own 8 query heads and 1
// KV head).  Flash-style (the CS336 lecture-8 book's activation-memory section:
// the s x s attention weights are recomputed from Q, K and the saved row
// log-sum-exp instead of being stored): with P = exp(Q K^T / sqrt(d) - lse),
//     dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO,
// and a KV head's dK, dV summed over the query heads that share it.
//
// Three launches, every sum in a fixed order (results are identical run to run):
//  1. attn_bwd_dq_kernel, query-major (the forward kernel's structure): a
//     workgroup of 8 wave64s takes query blocks i and nqb-1-i (equal causal
//     length); its two 4-wave groups split the key tiles in halves and add
//     their dQ partials through LDS.  Transposed products, as in the forward:
//     S^T = K Q^T and dP^T = V dO^T put one query column in each lane, so
//     lse, D and the rescale are per-lane scalars, and dS^T feeds
//     dQ^T += K^T dS^T straight from the accumulator registers (its keys in a
//     lane-local order that the K^T transpose reads follow).  Before its key
//     loop each wave computes D for its queries from dO and O, and writes the
//     base-2 lse and D of every query, padded to whole 64-query tiles, to the
//     workspace for launch 2.
//  2. attn_bwd_dkv_kernel, key-major: a workgroup owns one query head and the
//     key blocks i and nkb-1-i (128 keys each; equal causal length) and walks
//     the query tiles from each block's diagonal to the end.  Wave w holds keys
//     32 (w & 3) .. +31 of the block and queries 32 (w >> 2) .. +31 of each
//     64-query tile: S = Q K^T and dP = dO V^T put one key column in each lane
//     (P and dS then feed dV^T += dO^T P and dK^T += Q^T dS as the B operand
//     of a transposed product, in the lane-local query order the dO^T / Q^T
//     transpose reads follow).  The two query halves add their accumulators
//     through LDS, and the head's fp32 partial dK (unscaled) and dV go to the
//     workspace.
//  3. attn_bwd_reduce_kernel: each KV head's dK, dV = the sum of its query
//     heads' partials in increasing head order; dK scaled by 1/sqrt(d); bf16.
//
// Tiles are staged global -> LDS by buffer DMA (double-buffered query tiles).
// Q and dO tiles in launch 2 and the K tile in launch 1 are read both as
// 16-byte rows and through the LDS transpose read, so their 16-byte chunks
// are XOR-swizzled by dsw(r) = 4 (r & 3) + ((r >> 2) & 3): 16 consecutive rows
// put a chunk in 16 distinct places (row reads), and the 4 rows of one
// transpose read move a group of 4 aligned chunks to 4 disjoint groups.
#include "gemm_bf16_kernels.h"

namespace {

constexpr int HD = 128;                 // head dimension
constexpr int QBLK = 128;               // dQ kernel: query rows per workgroup
constexpr int KTL = 64;                 // dQ kernel: keys per tile
constexpr int KBLK = 128;               // dK/dV kernel: keys per block
constexpr int QTL = 64;                 // dK/dV kernel: queries per tile
constexpr int ROWB = HD * 2;            // bytes of one bf16 row of a head
constexpr float LOG2E = 1.4426950408889634f;

struct BwdArgs {
  const uint16_t *Q, *K, *V, *O, *dO;
  const float *lse;  // [nq][s], natural log-sum-exp of the forward
  float *stats;      // [nq][nqt][128]: base-2 lse of the tile's 64 queries, then their D
  float *pk, *pv;    // [nq][s][128] per-query-head partial dK (unscaled) and dV
  uint16_t *dQ, *dK, *dV;
  int s, nq, nkv, nqt;
  int64_t ldq, ldk;  // elements per row of Q / O / dO / dQ, of K / V / dK / dV
  float c;           // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
};

// chunk swizzles of a [rows][128] bf16 tile (256-byte rows)
__device__ __forceinline__ int rsw(int r) { return r & 15; }                       // 16-byte row reads only
__device__ __forceinline__ int dsw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }  // rows and transpose reads
__device__ __forceinline__ int roff(int r, int c) { return r * ROWB + ((c ^ rsw(r)) << 4); }
__device__ __forceinline__ int doff(int r, int c) { return r * ROWB + ((c ^ dsw(r)) << 4); }
// byte offset of element col of row r in a dsw-swizzled tile
__device__ __forceinline__ int delem(int r, int col) {
  return r * ROWB + (((col >> 3) ^ dsw(r)) << 4) + ((col & 7) << 1);
}

// ------------------------------------------------------------------ dQ (+ lse2, D)
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int TILE = KTL * ROWB;  // 16 KB: one K or V tile
  // [group][stage][K tile | V tile]
  __shared__ __attribute__((aligned(1024))) char sm[2][2][2 * TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wl = w & 3;
  const int h = lane >> 5, ql = lane & 31;
  const int head = blockIdx.x % a.nq;
  const int pair = blockIdx.x / a.nq;
  const int g = head / (a.nq / a.nkv);
  const int nqb = (a.s + QBLK - 1) / QBLK;
  char *const mine = sm[grp][0];
  float *const merge = (float *)sm[1][0];  // group 1's dQ partials: [4 waves][64 values][64 lanes]

  // DMA: in each group, wave wl stages kilobytes 4wl .. 4wl+3 of the K and the V tile
  uint32_t kvo[4], vvo[4];
  int krow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * wl + i, r = 4 * b + (lane >> 4), pos = lane & 15;
    krow[i] = r;
    kvo[i] = (uint32_t)(r * a.ldk * 2 + ((pos ^ dsw(r)) << 4));
    vvo[i] = (uint32_t)(r * a.ldk * 2 + ((pos ^ rsw(r)) << 4));
  }
  const uint32_t L0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sm[grp][0]));
  const uint32_t L1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sm[grp][1]));
  auto issue = [&](int t, uint32_t stage) {
    const int k0 = t * KTL;
    const i32x4 rk = rsrc_words(a.K + (int64_t)k0 * a.ldk + g * HD);
    const i32x4 rv = rsrc_words(a.V + (int64_t)k0 * a.ldk + g * HD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = k0 + krow[i] < a.s;
      dma16(rk, in ? kvo[i] : OOB, 0u, stage + (4 * wl + i) * 1024);
      dma16(rv, in ? vvo[i] : OOB, 0u, stage + TILE + (4 * wl + i) * 1024);
    }
  };

  // fragment offsets (stage-relative): K and V rows for S^T and dP^T (slice t of
  // key block kb at + kb * 32 rows: both swizzles repeat every 16 rows), K^T
  // transpose reads for dQ^T (d block db, 16-key slice tt at + tt * 16 rows):
  // rows 4h + (j >> 2) and 8 + 4h + (j >> 2) -- the key order of dS^T in this
  // lane's accumulator
  int ko[8], vo[8], kt[4][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    ko[t] = doff(ql, 2 * t + h);
    vo[t] = TILE + roff(ql, 2 * t + h);
  }
  {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      kt[db][0] = delem(4 * h + (j >> 2), col);
      kt[db][1] = delem(8 + 4 * h + (j >> 2), col);
    }
  }

  const int blocks[2] = {nqb - 1 - pair, pair};
  const int nblk = blocks[0] == blocks[1] ? 1 : 2;
  for (int bi = 0; bi < nblk; ++bi) {
    const int q0 = blocks[bi] * QBLK, qw0 = q0 + 32 * wl, myq = qw0 + ql;
    const bool qin = myq < a.s;
    // Q^T and dO^T fragments (slice t: d = 16t + 8h .. +7 of this lane's query),
    // and D = dO . O of the query: this half-lane's 64 products, then the other half's
    bf16x8 qf[8], df[8];
    float dsum = 0.f;
    {
      const int64_t ro = (int64_t)min(myq, a.s - 1) * a.ldq + head * HD + 8 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 vq = qin ? *(const u32x4 *)(a.Q + ro + 16 * t) : zero4();
        const u32x4 vd = qin ? *(const u32x4 *)(a.dO + ro + 16 * t) : zero4();
        const u32x4 vo_ = qin ? *(const u32x4 *)(a.O + ro + 16 * t) : zero4();
        qf[t] = __builtin_bit_cast(bf16x8, vq);
        df[t] = __builtin_bit_cast(bf16x8, vd);
        float x[8], y[8];
        unpack8(vd, x);
        unpack8(vo_, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) dsum = fmaf(x[i], y[i], dsum);
      }
    }
    const float D = dsum + __shfl_xor(dsum, 32, 64);
    const float lse2 = qin ? a.lse[(int64_t)head * a.s + myq] * LOG2E : INFINITY;
    if (grp == 0 && h == 0) {  // the key-major kernel's per-query statistics
      float *st = a.stats + ((int64_t)head * a.nqt + (myq >> 6)) * 128 + (myq & 63);
      st[0] = lse2;
      st[64] = qin ? D : 0.f;
    }

    const int kend = min(q0 + QBLK, a.s);  // keys the block needs: 0 .. kend - 1
    const int n = (kend + KTL - 1) / KTL;
    const int n0 = n / 2;
    const int tbeg = grp ? n0 : 0, tcnt = grp ? n - n0 : n0;
    const int iters = n - n0;              // >= n0: both groups pass the same barriers
    const int wkend = min(qw0 + 32, a.s);  // keys this wave needs
    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

    if (tcnt > 0) issue(tbeg, L0);
    for (int it = 0; it < iters; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (it + 1 < tcnt) issue(tbeg + it + 1, (it & 1) ? L0 : L1);
      const int k0 = (tbeg + it) * KTL;
      if (it >= tcnt || k0 >= wkend) continue;  // wave-uniform
      const char *S = mine + (it & 1) * 2 * TILE;

      // per 32-key block kb: S^T = K Q^T and dP^T = V dO^T, then
      // P = exp2(S c - lse2) and dS = P (dP - D) -- element e is key
      // k0 + 32 kb + 8 (e/4) + 4h + e%4, and keys after the query are masked on
      // the tiles that cross the wave's diagonal -- then dQ^T += K^T dS^T over
      // the block's two 16-key slices
      const bool diag = k0 + KTL - 1 > qw0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sa, pa;
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[e] = pa[e] = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + kb * 32 * ROWB + ko[t]));
          sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sa, 0, 0, 0);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + kb * 32 * ROWB + vo[t]));
          pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[t], pa, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float p = tp_exp2(fmaf(sa[e], a.c, -lse2));
          if (diag && k0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3) > myq) p = 0.f;
          sa[e] = p * (pa[e] - D);
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int tt = 2 * kb + t2;
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] = sa[8 * t2 + i];
          const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8(pv));
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x8 kf = read_tr(S + kt[db][0] + tt * 16 * ROWB, S + kt[db][1] + tt * 16 * ROWB);
            dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, pf, dq[db], 0, 0, 0);
          }
        }
      }
    }

    // group 1 hands its partial dQ^T to the group-0 wave with the same queries
    __syncthreads();
    if (grp == 1) {
      float *po = merge + wl * 64 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) po[(16 * db + e) * 64] = dq[db][e];
    }
    __syncthreads();
    if (grp == 0) {
      const float *po = merge + wl * 64 * 64 + lane;
      // dQ rows through LDS: this wave's [32 q][128 d] bf16, chunks XOR-swizzled by the row
      char *ob = sm[0][1] + wl * 8192;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (dq[db][4 * j4 + i] + po[(16 * db + 4 * j4 + i) * 64]) * a.scale;
#pragma unroll
          for (int i = 4; i < 8; ++i) v[i] = 0.f;
          const u32x4 pk = pack8(v);
          uint2 two;
          two.x = pk[0];
          two.y = pk[1];
          *(uint2 *)(ob + ql * 256 + (((4 * db + j4) ^ (ql & 15)) << 4) + 8 * h) = two;
        }
      // each wave reads back only its own strip (a wave's LDS operations complete in order)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int idx = it * 64 + lane, r = idx >> 4, c = idx & 15;
        const u32x4 v = *(const u32x4 *)(ob + r * 256 + ((c ^ (r & 15)) << 4));
        if (qw0 + r < a.s) *(u32x4 *)(a.dQ + (int64_t)(qw0 + r) * a.ldq + head * HD + c * 8) = v;
      }
    }
    __syncthreads();  // LDS is reused by the next block
  }
}

// ------------------------------------------------------------------ dK, dV partials
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkv_kernel(BwdArgs a) {
  constexpr int KVT = KBLK * ROWB;   // 32 KB: the block's K or V
  constexpr int QT = QTL * ROWB;     // 16 KB: one Q or dO tile
  constexpr int STG = 2 * QT + 1024; // a stage: Q tile, dO tile, [lse2 x 64 | D x 64]
  __shared__ __attribute__((aligned(1024))) char sm[2 * KVT + 2 * STG];
  char *const sK = sm, *const sV = sm + KVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = w & 3, qh = w >> 2;
  const int h = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x % a.nq;
  const int pair = blockIdx.x / a.nq;
  const int g = head / (a.nq / a.nkv);
  const int nkb = (a.s + KBLK - 1) / KBLK;
  const int nqt = (a.s + QTL - 1) / QTL;

  // DMA lane offsets: the block's K and V (128 rows: kilobytes 4w .. 4w+3 of each),
  // a Q / dO tile (64 rows: kilobytes 2w, 2w+1 of each)
  uint32_t kvo[4], qdo[2];
  int kr[4], qr[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (4 * w + i) + (lane >> 4), pos = lane & 15;
    kr[i] = r;
    kvo[i] = (uint32_t)(r * a.ldk * 2 + ((pos ^ rsw(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * w + i) + (lane >> 4), pos = lane & 15;
    qr[i] = r;
    qdo[i] = (uint32_t)(r * a.ldq * 2 + ((pos ^ dsw(r)) << 4));
  }
  const uint32_t LK = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sK));
  const uint32_t LS0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(sm + 2 * KVT));
  const uint32_t LS1 = LS0 + STG;
  auto issue_kv = [&](int k0) {
    const i32x4 rk = rsrc_words(a.K + (int64_t)k0 * a.ldk + g * HD);
    const i32x4 rv = rsrc_words(a.V + (int64_t)k0 * a.ldk + g * HD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = k0 + kr[i] < a.s;
      dma16(rk, in ? kvo[i] : OOB, 0u, LK + (4 * w + i) * 1024);
      dma16(rv, in ? kvo[i] : OOB, 0u, LK + KVT + (4 * w + i) * 1024);
    }
  };
  auto issue_q = [&](int qt, uint32_t stage) {
    const int q0 = qt * QTL;
    const i32x4 rq = rsrc_words(a.Q + (int64_t)q0 * a.ldq + head * HD);
    const i32x4 rd = rsrc_words(a.dO + (int64_t)q0 * a.ldq + head * HD);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool in = q0 + qr[i] < a.s;
      dma16(rq, in ? qdo[i] : OOB, 0u, stage + (2 * w + i) * 1024);
      dma16(rd, in ? qdo[i] : OOB, 0u, stage + QT + (2 * w + i) * 1024);
    }
    if (w == 0) {  // 512 bytes of statistics (lanes 32..63 fill the rest of the kilobyte with zeros)
      const i32x4 rs = rsrc_words(a.stats + ((int64_t)head * a.nqt + qt) * 128);
      dma16(rs, lane < 32 ? (uint32_t)(lane * 16) : OOB, 0u, stage + 2 * QT);
    }
  };

  // fragment offsets (relative to the stage / the K and V region):
  //  S = Q K^T, dP = dO V^T: A = rows 32 qh + l32 of the Q / dO tile (slice t),
  //  B = rows 32 ks + l32 of K / V;
  //  dV^T += dO^T P, dK^T += Q^T dS: A through transpose reads of the dO / Q tile
  //  (d block db, 16-query slice tt at + tt * 16 rows), rows 32 qh + 4h + (j >> 2)
  //  and 32 qh + 8 + 4h + (j >> 2) -- the query order of P and dS in this lane
  int qo[8], ko[8], tr[4][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    qo[t] = doff(32 * qh + l32, 2 * t + h);
    ko[t] = roff(32 * ks + l32, 2 * t + h);
  }
  {
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      tr[db][0] = delem(32 * qh + 4 * h + (j >> 2), col);
      tr[db][1] = delem(32 * qh + 8 + 4 * h + (j >> 2), col);
    }
  }

  const int blocks[2] = {pair, nkb - 1 - pair};
  const int nblk = blocks[0] == blocks[1] ? 1 : 2;
  for (int bi = 0; bi < nblk; ++bi) {
    const int kb0 = blocks[bi] * KBLK, kw0 = kb0 + 32 * ks, mykey = kw0 + l32;
    const int qt0 = kb0 / QTL, ntile = nqt - qt0;
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

    issue_kv(kb0);
    issue_q(qt0, LS0);
    for (int it = 0; it < ntile; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (it + 1 < ntile) issue_q(qt0 + it + 1, (it & 1) ? LS0 : LS1);
      const int qw0 = (qt0 + it) * QTL + 32 * qh;
      if (qw0 + 31 < kw0) continue;  // every key of the wave after every query (wave-uniform)
      const char *S = sm + 2 * KVT + (it & 1) * STG;
      const float *st = (const float *)(S + 2 * QT);

      f32x16 sa, pa;
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[e] = pa[e] = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 qf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + qo[t]));
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sK + ko[t]));
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf, sa, 0, 0, 0);
        const bf16x8 df = __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + QT + qo[t]));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sV + ko[t]));
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df, vf, pa, 0, 0, 0);
      }
      // element e is query qw0 + 8 (e/4) + 4h + e%4 of this lane's key: its base-2
      // lse and D come four at a time from the stage's statistics (queries past
      // the sequence carry lse2 = +inf, so their P is 0); keys after the query are
      // masked on the tiles that cross the wave's diagonal
      const bool diag = qw0 < kw0 + 31;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 l4 = *(const float4 *)(st + 32 * qh + 8 * m + 4 * h);
        const float4 d4 = *(const float4 *)(st + 64 + 32 * qh + 8 * m + 4 * h);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * m + i;
          float p = tp_exp2(fmaf(sa[e], a.c, -lv[i]));
          if (diag && mykey > qw0 + 8 * m + 4 * h + i) p = 0.f;
          sa[e] = p;
          pa[e] = p * (pa[e] - dd[i]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over two 16-query slices
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float pv[8], sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = sa[8 * tt + i];
          sv[i] = pa[8 * tt + i];
        }
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8(pv));
        const bf16x8 sf = __builtin_bit_cast(bf16x8, pack8(sv));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 of = read_tr(S + QT + tr[db][0] + tt * 16 * ROWB, S + QT + tr[db][1] + tt * 16 * ROWB);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, pf, dv[db], 0, 0, 0);
          const bf16x8 qf = read_tr(S + tr[db][0] + tt * 16 * ROWB, S + tr[db][1] + tt * 16 * ROWB);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, sf, dk[db], 0, 0, 0);
        }
      }
    }

    // The two query halves add their accumulators in a fixed order (half 0 +
    // half 1): half 1 hands over dV, half 0 hands over dK, through LDS laid out
    // [ks][value][lane]; half 0 then writes dV, half 1 dK.  Element e of d block
    // db is d = 32 db + 8 (e/4) + 4h + e%4 of key mykey: four consecutive floats.
    __syncthreads();
    {
      float *xo = (float *)sm + (qh ? 0 : 64 * 64 * 4) + ks * 64 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xo[(16 * db + e) * 64] = qh ? dv[db][e] : dk[db][e];
    }
    __syncthreads();
    {
      const float *xi = (const float *)sm + (qh ? 64 * 64 * 4 : 0) + ks * 64 * 64 + lane;
      float *part = (qh ? a.pk : a.pv) + ((int64_t)head * a.s + mykey) * HD + 4 * h;
      if (mykey < a.s) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * m + i;
              const float other = xi[(16 * db + e) * 64];
              o[i] = qh ? other + dk[db][e] : dv[db][e] + other;
            }
            *(float4 *)(part + 32 * db + 8 * m) = make_float4(o[0], o[1], o[2], o[3]);
          }
      }
    }
    __syncthreads();  // LDS is reused by the next block
  }
}

// ------------------------------------------------------------------ reduce over each group's heads
// Thread: 8 consecutive d of one key of one KV head, for dK (first half of the
// grid) or dV.  Sums the group's query-head partials in increasing head order.
__global__ void __launch_bounds__(256) attn_bwd_reduce_kernel(BwdArgs a) {
  const int64_t runs = (int64_t)a.s * a.nkv * (HD / 8);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * runs) return;
  const bool isv = idx >= runs;
  const int64_t r = isv ? idx - runs : idx;
  const int c8 = (int)(r % (HD / 8));
  const int64_t rk = r / (HD / 8);
  const int gk = (int)(rk % a.nkv);
  const int64_t key = rk / a.nkv;
  const int grp = a.nq / a.nkv;
  const float *part = isv ? a.pv : a.pk;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = gk * grp; j < (gk + 1) * grp; ++j) {
    const float4 *p = (const float4 *)(part + ((int64_t)j * a.s + key) * HD + 8 * c8);
    const float4 x = p[0], y = p[1];
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
    acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
  }
  if (!isv) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= a.scale;
  }
  uint16_t *out = (isv ? a.dV : a.dK) + key * a.ldk + gk * HD + 8 * c8;
  *(u32x4 *)out = pack8(acc);
}

}  // namespace

size_t tp_attn_bwd_ws_bytes(int64_t s, int64_t nq) {
  const int64_t nqt = (s + QBLK - 1) / QBLK * (QBLK / QTL);
  const size_t stats = ((size_t)nq * nqt * 128 * sizeof(float) + 255) & ~size_t(255);
  const size_t part = ((size_t)nq * s * HD * sizeof(float) + 255) & ~size_t(255);
  return stats + 2 * part;
}

hipError_t tp_launch_attn_bwd(int64_t s, int64_t nq, int64_t nkv, const void *Q, const void *K, const void *V,
                              const void *O, const void *dO, const float *lse, void *dQ, void *dK, void *dV,
                              void *ws, hipStream_t st) {
  if (s == 0 || nq == 0) return hipSuccess;
  BwdArgs a;
  a.Q = (const uint16_t *)Q;
  a.K = (const uint16_t *)K;
  a.V = (const uint16_t *)V;
  a.O = (const uint16_t *)O;
  a.dO = (const uint16_t *)dO;
  a.lse = lse;
  a.s = (int)s;
  a.nq = (int)nq;
  a.nkv = (int)nkv;
  a.nqt = (int)((s + QBLK - 1) / QBLK * (QBLK / QTL));
  const size_t stats = ((size_t)nq * a.nqt * 128 * sizeof(float) + 255) & ~size_t(255);
  const size_t part = ((size_t)nq * s * HD * sizeof(float) + 255) & ~size_t(255);
  a.stats = (float *)ws;
  a.pk = (float *)((char *)ws + stats);
  a.pv = (float *)((char *)ws + stats + part);
  a.dQ = (uint16_t *)dQ;
  a.dK = (uint16_t *)dK;
  a.dV = (uint16_t *)dV;
  a.ldq = nq * HD;
  a.ldk = nkv * HD;
  a.scale = 1.f / sqrtf((float)HD);
  a.c = LOG2E * a.scale;
  const int64_t nqb = (s + QBLK - 1) / QBLK, nkb = (s + KBLK - 1) / KBLK;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)((nqb + 1) / 2 * nq)), dim3(512), 0, st, a);
  hipLaunchKernelGGL(attn_bwd_dkv_kernel, dim3((unsigned)((nkb + 1) / 2 * nq)), dim3(512), 0, st, a);
  const int64_t threads = 2 * s * nkv * (HD / 8);
  hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}
