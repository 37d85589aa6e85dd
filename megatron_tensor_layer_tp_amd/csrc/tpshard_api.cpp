// tpshard_api.cpp -- the extern "C" entry points of libtpshard.
//
// Each call validates every argument before anything is enqueued, plans the
// launch (tile shape, split-K) from the sizes alone -- so the workspace size
// queries and the calls agree -- and enqueues its kernels on the caller's
// stream.  No allocation, no state beyond the per-thread error string.
//
// The operations are those of the pages: column- and row-parallel products
// and the two-card worked example (book "7.3 模型并行与张量并行" §7.3.2),
// the backward pass (§7.3.3), attention/SwiGLU/vocab sharding (§7.3.4), and
// the fused vocab-parallel cross entropy (lecture 16 notes §5.5).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>
#include <string>

#include "../../include/tpshard.h"
#include "gemm_desc.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(tp_status_string(code)) + ": " + buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return TP_OK;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int kCUs = 256;     // MI355X compute units
constexpr int kBK = 64;       // K tile of both GEMM paths

// ---------------------------------------------------------------- checks
struct Checker {
  int status = TP_OK;
  bool dim(int64_t v, const char *name) {
    if (status) return false;
    if (v < 0 || v > kMaxDim) {
      status = fail(TP_ESHAPE, "%s = %lld is negative or >= 2^31", name, (long long)v);
      return false;
    }
    return true;
  }
  // a pointer may be NULL only when its tensor has no elements
  bool ptr(const void *p, int64_t nelem, const char *name) {
    if (status) return false;
    if (nelem > 0 && p == nullptr) {
      status = fail(TP_EINVAL, "%s is NULL", name);
      return false;
    }
    if (((uintptr_t)p & 15) != 0) {
      status = fail(TP_EALIGN, "%s = %p is not 16-byte aligned", name, p);
      return false;
    }
    return true;
  }
  bool dtype(int dt, bool f32_ok, const char *call) {
    if (status) return false;
    if (dt != TP_DT_F32 && dt != TP_DT_BF16) {
      status = fail(TP_EINVAL, "%s: dtype %d is not a tp_dtype", call, dt);
      return false;
    }
    if (dt == TP_DT_F32 && !f32_ok) {
      status = fail(TP_EUNSUPPORTED, "%s: fp32 storage is not supported", call);
      return false;
    }
    return true;
  }
  bool act(int a) {
    if (status) return false;
    if (a != TP_ACT_RELU && a != TP_ACT_GELU) {
      status = fail(TP_EINVAL, "act %d is not a tp_act", a);
      return false;
    }
    return true;
  }
  bool elems(int64_t a, int64_t b, int64_t &out, const char *what) {
    if (status) return false;
    if (a != 0 && b > INT64_MAX / 8 / a) {
      status = fail(TP_ESHAPE, "%s has too many elements", what);
      return false;
    }
    out = a * b;
    return true;
  }
};

// Scratch of the allocation-free fused LM head + CE call
// (tp_lm_head_ce_fwd_noalloc): a file-scope device array, 32 MiB, of which each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array: kernels get
// the per-device address hipGetSymbolAddress returns, fetched once per device
// with that device current (scratch_ptr below).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
}  // namespace
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
namespace {

// ---------------------------------------------------------------- planning
struct Plan {
  int bm = 128, bn = 128, res = RES_THREE, splits = 1, kt_per_split = 1, tiles_m = 0, tiles_n = 0;
  bool vec = true;
  size_t ws_bytes = 0;  // split-K partials
};

struct Spec {               // one product, described before planning
  int layout = GEMM_NN;
  int epi = EPI_STORE;
  bool out_f32 = false;
  int64_t M = 0, K = 0;     // K = total when kseg
  int nseg = 1;
  bool kseg = false;
  bool dual = false;
  bool can_split = false;   // a workspace for split-K partials is available
  int64_t seg[TP_MAX_SEG] = {0, 0, 0};  // N-extents (N-segments) or K-extents (K-segments)
  int64_t N = 0;            // total N (kseg or single segment)
  int64_t lds[12] = {};     // every leading dimension involved
  int nlds = 0;
  void ld(int64_t v) { lds[nlds++] = v; }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t ntiles_n(const Spec &s, int bn) {
  if (s.kseg) return cdiv(s.N, bn);
  const int w = s.dual ? bn / 2 : bn;
  int64_t t = 0;
  for (int i = 0; i < s.nseg; ++i) t += cdiv(s.seg[i], w);
  return t;
}

int64_t ktiles(const Spec &s) {
  if (!s.kseg) return cdiv(s.K, kBK);
  int64_t t = 0;
  for (int i = 0; i < s.nseg; ++i) t += cdiv(s.seg[i], kBK);
  return t;
}

// ---- cost model of the bf16 DMA kernels (microseconds, measured on MI355X)
// For each built (tile, residency) variant: the time of one 64-deep K step of a
// block when every slot of its CU is busy (`step`), the same over launches of
// three or more rounds (`step_long`: two workgroups per CU then lose more to
// L2 misses), and when a two-workgroup variant has its CU to itself
// (`alone`); the per-block prologue + bf16-store epilogue (`fixed`); and the
// extra cost of the first round of a launch (`first`).  Fitted from K sweeps
// of one- and two-round NN products and from full products of K = 8192.
struct TileCost {
  int bm, bn, res;
  double step, step_long, alone, fixed, first;
};
constexpr TileCost kTiles[] = {
    {256, 256, RES_WAVES8, 1.53, 1.53, 1.53, 11.3, 1.2},  {256, 256, RES_TWO, 1.58, 1.58, 1.58, 11.3, 1.2},
    {256, 192, RES_TWO, 1.26, 1.26, 1.26, 10.0, 1.0},
    {256, 128, RES_THREE, 0.91, 0.91, 0.91, 10.0, 0.5},   {128, 256, RES_THREE, 0.91, 0.91, 0.91, 10.0, 0.7},
    {128, 192, RES_THREE, 0.72, 0.72, 0.72, 7.8, 1.6},    {128, 128, RES_THREE, 0.57, 0.57, 0.57, 6.0, 0.3},
    {128, 192, RES_SHARED, 1.15, 1.60, 0.78, 5.4, 9.6},   {128, 128, RES_SHARED, 0.975, 1.35, 0.65, 3.2, 3.6},
};
constexpr double kLaunchUs = 2.0;     // one more kernel in the stream
constexpr double kReduceBw = 4.0e6;   // split-K reduction traffic, bytes per microsecond

// extra epilogue time per output element of a block, beyond a bf16 store
double epi_cost(int epi, bool out_f32, int res) {
  const bool sh = res == RES_SHARED;
  switch (epi) {
  case EPI_ACT_FWD: return sh ? 1.3e-4 : 1.7e-4;
  case EPI_ACT_BWD: return sh ? 2.4e-4 : 2.9e-4;
  case EPI_SWIGLU_FWD: return sh ? 1.6e-4 : 2.0e-4;
  case EPI_SWIGLU_BWD: return sh ? 3.3e-4 : 4.0e-4;
  case EPI_PARTIAL: return sh ? 0.3e-4 : 0.7e-4;
  case EPI_CE_STATS: return 1.0e-4;
  default: return out_f32 ? (sh ? 0.2e-4 : 0.5e-4) : 0.0;
  }
}

bool variant_built(int bm, int bn, int res, bool dual, int epi) {
  if (bn == 192 && (dual || epi == EPI_CE_STATS)) return false;
  for (const TileCost &t : kTiles)
    if (t.bm == bm && t.bn == bn && t.res == res) return true;
  return false;
}
const TileCost &tile_cost(int bm, int bn, int res) {
  for (const TileCost &t : kTiles)
    if (t.bm == bm && t.bn == bn && t.res == res) return t;
  return kTiles[0];
}

// duration of one block of the planned product (kps K steps) in a launch of
// `nb` blocks in all
double block_us(const Spec &s, const Plan &p, int64_t nb) {
  const TileCost &t = tile_cost(p.bm, p.bn, p.res);
  const int64_t slots = (int64_t)kCUs * res_wgs(p.res);
  const double step = nb <= kCUs ? t.alone : (nb > 2 * slots ? t.step_long : t.step);
  const int epi = p.splits > 1 ? (int)EPI_PARTIAL : s.epi;
  return p.kt_per_split * step + t.fixed + epi_cost(epi, p.splits > 1 || s.out_f32, p.res) * p.bm * p.bn;
}
int64_t plan_blocks(const Plan &p) { return (int64_t)p.tiles_m * p.tiles_n * p.splits; }
int plan_slots(const Plan &p) { return kCUs * res_wgs(p.res); }

// the split-K reduction pass: read every partial, write the output
double reduce_us(const Spec &s, const Plan &p) {
  if (p.splits <= 1) return 0.0;
  const double bytes = (double)s.M * s.N * (4.0 * p.splits + (s.out_f32 ? 4.0 : 2.0));
  return kLaunchUs + bytes / kReduceBw;
}

// greedy dispatch of n1 blocks of d1 then n2 blocks of d2 over `slots`
// workgroup slots (each new block to the earliest free slot): the makespan.
// Slots free at the same time are handled as one group, so the loop runs about
// once per round.
double list_makespan(int64_t n1, double d1, int64_t n2, double d2, int slots) {
  std::map<double, int64_t> free_at{{0.0, slots}};
  double end = 0.0;
  auto run = [&](int64_t n, double d) {
    while (n > 0) {
      const auto it = free_at.begin();
      const double t = it->first;
      const int64_t c = it->second;
      free_at.erase(it);
      const int64_t k = std::min(c, n);
      n -= k;
      if (c > k) free_at[t] += c - k;
      free_at[t + d] += k;
      end = std::max(end, t + d);
    }
  };
  run(n1, d1);
  run(n2, d2);
  return end;
}

// estimated time of one planned product launched alone (with its reduction)
double plan_us(const Spec &s, const Plan &p) {
  const int64_t nb = plan_blocks(p);
  if (nb == 0) return 0.0;
  const int slots = plan_slots(p);
  const double d = block_us(s, p, nb);
  const double rounds = (double)((nb + slots - 1) / slots);
  return kLaunchUs + tile_cost(p.bm, p.bn, p.res).first + rounds * d + reduce_us(s, p);
}

// TP_GEMM_VARIANT="BMxBN:two|three|shared|waves8" restricts every bf16 product that has
// that variant built (and 16-byte operands) to it, split counts still chosen by
// the cost model; the parity tests use it to run each variant on the same sizes.
struct ForcedVariant {
  bool on = false;
  int bm = 0, bn = 0, res = 0;
};
ForcedVariant forced_variant() {
  ForcedVariant f;
  const char *e = std::getenv("TP_GEMM_VARIANT");
  if (e == nullptr || *e == 0) return f;
  char r[16] = {0};
  if (std::sscanf(e, "%dx%d:%15s", &f.bm, &f.bn, r) != 3) return f;
  const std::string rs(r);
  f.res = rs == "two" ? RES_TWO : rs == "three" ? RES_THREE : rs == "shared" ? RES_SHARED
         : rs == "waves8" ? RES_WAVES8 : -1;
  f.on = f.res >= 0;
  return f;
}

// every built variant of the product with the split counts worth trying
template <class F>
void for_each_plan(const Spec &s, F &&f) {
  bool vec = true;
  // 16-byte DMA / buffer loads: leading dimensions multiples of 8 elements, and
  // a 256-row tile's byte span addressable with 32-bit buffer offsets
  for (int i = 0; i < s.nlds; ++i) vec &= s.lds[i] % 8 == 0 && s.lds[i] < (int64_t(1) << 21);
  vec &= s.M % 8 == 0;
  if (s.kseg) {
    vec &= s.N % 8 == 0;
    for (int i = 0; i < s.nseg; ++i) vec &= s.seg[i] % 8 == 0;
  } else {
    vec &= s.K % 8 == 0;
    for (int i = 0; i < s.nseg; ++i) vec &= s.seg[i] % 8 == 0;
  }
  const int64_t KT = ktiles(s);
  const bool can_split = s.can_split && s.epi == EPI_STORE && !s.dual && KT >= 8;
  ForcedVariant fv = forced_variant();
  if (fv.on && !(vec && variant_built(fv.bm, fv.bn, fv.res, s.dual, s.epi))) fv.on = false;
  for (const TileCost &t : kTiles) {
    if (fv.on && !(t.bm == fv.bm && t.bn == fv.bn && t.res == fv.res)) continue;
    Plan p;
    p.vec = vec;
    p.bm = t.bm;
    p.bn = t.bn;
    p.res = t.res;
    if (!vec) {  // the element-wise kernel: 128x128, one workgroup per CU
      if (!(t.bm == 128 && t.bn == 128 && t.res == RES_THREE)) continue;
    } else if (!variant_built(t.bm, t.bn, t.res, s.dual, s.epi)) {
      continue;
    }
    p.tiles_m = (int)cdiv(s.M, p.bm);
    p.tiles_n = (int)ntiles_n(s, p.bn);
    for (int sp = 1; sp <= (can_split && vec ? 16 : 1); ++sp) {
      const int64_t kps = cdiv(std::max<int64_t>(KT, 1), sp);
      if (sp > 1 && (kps < 4 || cdiv(KT, kps) < sp)) break;
      p.splits = sp;
      p.kt_per_split = (int)kps;
      p.ws_bytes = sp > 1 ? (size_t)sp * s.M * s.N * sizeof(float) : 0;
      f(p);
    }
  }
}

Plan plan_bf16(const Spec &s) {
  Plan best;
  double best_t = 1e300;
  for_each_plan(s, [&](const Plan &p) {
    const double t = plan_us(s, p);
    if (t < best_t * 0.999) {
      best_t = t;
      best = p;
    }
  });
  return best;
}

Plan plan_f32(const Spec &s) {
  Plan p;
  p.bm = p.bn = TP_F32_TILE;
  p.tiles_m = (int)cdiv(s.M, TP_F32_TILE);
  int64_t tn = 0;
  if (s.kseg) tn = cdiv(s.N, TP_F32_TILE);
  else
    for (int i = 0; i < s.nseg; ++i) tn += cdiv(s.seg[i], TP_F32_TILE);
  p.tiles_n = (int)tn;
  p.splits = 1;
  p.kt_per_split = (int)std::max<int64_t>(ktiles(s), 1);
  return p;
}

Plan plan(const Spec &s, int dt) { return dt == TP_DT_BF16 ? plan_bf16(s) : plan_f32(s); }

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Build the kernel descriptor for a spec + plan and launch it (plus the
// split-K reduction).  Pointers: A[i], B[i], C[i] per segment.
struct Ptrs {
  const void *A[TP_MAX_SEG] = {};
  int64_t lda[TP_MAX_SEG] = {};
  const void *B[TP_MAX_SEG] = {};
  int64_t ldb[TP_MAX_SEG] = {};
  void *C[TP_MAX_SEG] = {};
  int64_t ldc[TP_MAX_SEG] = {};
  const void *ai0 = nullptr, *ai1 = nullptr;
  int64_t ldai = 0;
  void *ao0 = nullptr, *ao1 = nullptr;
  int64_t ldao = 0;
  int act = ACT_RELU;
  int stream_out = 0;  // GemmDesc::stream_out
};

// tile rows per group of the launch's tile order (the kernels walk a group's
// columns, XCD by XCD)
constexpr int kGroupM = 8;

GemmDesc make_desc(const Spec &s, const Ptrs &q, const Plan &p, int dt, void *ws) {
  GemmDesc d;
  std::memset(&d, 0, sizeof d);
  d.M = (int32_t)s.M;
  d.K = (int32_t)s.K;
  d.nseg = s.nseg;
  d.kseg = s.kseg;
  d.dual = s.dual;
  d.act = q.act;
  int64_t col = 0, tile = 0;
  const int wn = (s.dual && dt == TP_DT_BF16) ? p.bn / 2 : p.bn;
  for (int i = 0; i < s.nseg; ++i) {
    d.seg_len[i] = (int32_t)s.seg[i];
    d.seg_col0[i] = (int32_t)col;
    d.seg_tile0[i] = (int32_t)tile;
    col += s.seg[i];
    tile += s.kseg ? cdiv(s.seg[i], kBK) : cdiv(s.seg[i], wn);
  }
  d.seg_tile0[s.nseg] = (int32_t)tile;
  d.N = (int32_t)(s.kseg ? s.N : (s.dual ? s.seg[0] : col));
  for (int i = 0; i < TP_MAX_SEG; ++i) {
    d.A[i] = q.A[i];
    d.lda[i] = q.lda[i];
    d.B[i] = q.B[i];
    d.ldb[i] = q.ldb[i];
    d.C[i] = q.C[i];
    d.ldc[i] = q.ldc[i];
  }
  d.ai0 = q.ai0;
  d.ai1 = q.ai1;
  d.ldai = q.ldai;
  d.ao0 = q.ao0;
  d.ao1 = q.ao1;
  d.ldao = q.ldao;
  d.splits = p.splits;
  d.kt_per_split = p.kt_per_split;
  d.tiles_m = p.tiles_m;
  d.tiles_n = p.tiles_n;
  d.group_m = kGroupM;
  d.ws = (float *)ws;
  d.stream_out = q.stream_out;
  return d;
}

// the kernel variant a bf16 plan launches (split-K plans write fp32 partials)
GemmVariant variant(const Spec &s, const Plan &p) {
  GemmVariant v;
  v.layout = s.layout;
  v.epi = p.splits > 1 ? (int)EPI_PARTIAL : s.epi;
  v.out_f32 = p.splits > 1 ? true : s.out_f32;
  v.bm = p.bm;
  v.bn = p.bn;
  v.res = p.res;
  v.vec = p.vec;
  return v;
}

// Host replica of the kernels' logical tile order (tile_of, group_m tile rows
// per group, columns within a group): logical tile t -> (tile row, tile column).
void tile_rc(int tiles_m, int tiles_n, int group_m, int t, int &tm, int &tn) {
  const int in_group = group_m * tiles_n;
  const int g = t / in_group;
  const int first = g * group_m;
  const int gsz = std::min(tiles_m - first, group_m);
  const int w = t - g * in_group;
  tm = first + w % gsz;
  tn = w / gsz;
}

// The last round of a launch that fills at most half the workgroup slots,
// re-tiled: the first launch runs only the whole rounds (a prefix of the tile
// order: the kernels map block ids onto [0, grid)), and the remaining tiles,
// when they form a rectangle of the output, run as a product of their own
// with the tile shape the planner picks for that sub-matrix (smaller tiles
// spread it over all the slots).  Same epilogue, same K, no workspace.
struct Tail {
  bool on = false;
  int head = 0;                 // blocks of the first launch
  int64_t r0 = 0, c0 = 0;       // first output row and column of the rectangle
  Spec sub;
  Plan p;
};

// TP_GEMM_TAIL=off never re-tiles a last round; =force re-tiles it whenever it
// is a rectangle of at most half the slots, whatever the cost model says (the
// parity tests use it to run the path at small sizes); unset: the cost model decides.
int tail_mode() {
  const char *e = std::getenv("TP_GEMM_TAIL");
  if (e == nullptr) return 0;
  if (std::strcmp(e, "off") == 0) return -1;
  if (std::strcmp(e, "force") == 0) return 1;
  return 0;
}

Tail plan_tail(const Spec &s, const Plan &p) {
  Tail t;
  const int mode = tail_mode();
  if (mode < 0 || !p.vec || p.splits != 1 || s.nseg != 1 || s.kseg || s.epi == EPI_CE_STATS) return t;
  const int T = p.tiles_m * p.tiles_n, S = plan_slots(p);
  const int rem = T % S;
  if (T <= S || rem == 0 || 2 * rem > S) return t;
  int a = p.tiles_m, b = -1, c = p.tiles_n, e = -1;
  for (int i = T - rem; i < T; ++i) {
    int tm, tn;
    tile_rc(p.tiles_m, p.tiles_n, kGroupM, i, tm, tn);
    a = std::min(a, tm);
    b = std::max(b, tm);
    c = std::min(c, tn);
    e = std::max(e, tn);
  }
  if ((int64_t)(b - a + 1) * (e - c + 1) != rem) return t;
  const int ncols = s.dual ? p.bn / 2 : p.bn;
  Spec sub = s;
  sub.can_split = false;
  sub.M = std::min<int64_t>((int64_t)(b + 1) * p.bm, s.M) - (int64_t)a * p.bm;
  sub.N = std::min<int64_t>((int64_t)(e + 1) * ncols, s.seg[0]) - (int64_t)c * ncols;
  sub.seg[0] = sub.N;
  const Plan p2 = plan_bf16(sub);
  if (!p2.vec || p2.splits != 1) return t;
  const int head = T - rem;
  const double head_us = kLaunchUs + tile_cost(p.bm, p.bn, p.res).first + (double)(head / S) * block_us(s, p, head);
  if (mode == 0 && head_us + plan_us(sub, p2) >= 0.98 * plan_us(s, p)) return t;
  t.on = true;
  t.head = head;
  t.r0 = (int64_t)a * p.bm;
  t.c0 = (int64_t)c * ncols;
  t.sub = sub;
  t.p = p2;
  return t;
}

// the operand and output pointers of the sub-matrix at (r0, c0) of a product
Ptrs offset_ptrs(const Spec &s, const Ptrs &q, int64_t r0, int64_t c0) {
  Ptrs o = q;
  const int64_t cb = s.out_f32 ? 4 : 2;
  auto adv = [](const void *p, int64_t bytes) { return (const void *)((const char *)p + bytes); };
  o.A[0] = adv(q.A[0], 2 * (s.layout == GEMM_TN ? r0 : r0 * q.lda[0]));
  for (int i = 0; i < (s.dual ? 2 : 1); ++i)
    o.B[i] = adv(q.B[i], 2 * (s.layout == GEMM_NT ? c0 * q.ldb[i] : c0));
  o.C[0] = (void *)adv(q.C[0], cb * (r0 * q.ldc[0] + c0));
  if (q.ai0) o.ai0 = adv(q.ai0, 2 * (r0 * q.ldai + c0));
  if (q.ai1) o.ai1 = adv(q.ai1, 2 * (r0 * q.ldai + c0));
  if (q.ao0) o.ao0 = (void *)adv(q.ao0, 2 * (r0 * q.ldao + c0));
  if (q.ao1) o.ao1 = (void *)adv(q.ao1, 2 * (r0 * q.ldao + c0));
  return o;
}

// TP_PLAN_LOG=1: one line per launch on stderr with the plan the cost model chose
bool plan_log() {
  static const bool on = [] {
    const char *e = std::getenv("TP_PLAN_LOG");
    return e != nullptr && *e != 0 && *e != '0';
  }();
  return on;
}
const char *res_name(int res) {
  return res == RES_TWO ? "two" : res == RES_THREE ? "three" : res == RES_SHARED ? "shared" : "waves8";
}
void log_plan(const char *what, const Spec &s, const Plan &p, const char *extra = "") {
  if (!plan_log()) return;
  std::fprintf(stderr, "[tp plan] %s: M=%lld N=%lld K=%lld %dx%d:%s tiles=%dx%d splits=%d%s%s\n", what,
               (long long)s.M, (long long)s.N, (long long)s.K, p.bm, p.bn, res_name(p.res), p.tiles_m, p.tiles_n,
               p.splits, p.vec ? "" : " (element-wise loads)", extra);
}

int run_planned(const Spec &s, const Plan &p, const Ptrs &q, int dt, void *ws, hipStream_t st,
                const char *what) {
  if (p.splits > 1 && ws == nullptr) return fail(TP_EWORKSPACE, "%s: split-K plan without workspace", what);
  GemmDesc d = make_desc(s, q, p, dt, ws);
  hipError_t e;
  if (dt == TP_DT_F32) {
    e = tp_launch_gemm_f32(d, s.layout, s.epi, st);
  } else {
    const Tail tail = plan_tail(s, p);
    if (tail.on) d.nblocks = tail.head;
    if (plan_log()) {
      char extra[160] = "";
      if (tail.on)
        std::snprintf(extra, sizeof extra, "; first %d blocks, then rows %lld.. cols %lld.. (%lldx%lld) as %dx%d:%s",
                      tail.head, (long long)tail.r0, (long long)tail.c0, (long long)tail.sub.M,
                      (long long)tail.sub.N, tail.p.bm, tail.p.bn, res_name(tail.p.res));
      log_plan(what, s, p, extra);
    }
    const GemmVariant v = variant(s, p);
    e = tp_launch_gemm_bf16(d, v, st);
    if (e == hipSuccess && p.splits > 1) e = tp_launch_splitk_reduce(d, s.out_f32, p.vec, st);
    if (e == hipSuccess && tail.on) {
      const GemmDesc d2 = make_desc(tail.sub, offset_ptrs(s, q, tail.r0, tail.c0), tail.p, dt, nullptr);
      e = tp_launch_gemm_bf16(d2, variant(tail.sub, tail.p), st);
    }
  }
  if (e != hipSuccess) return fail(TP_EHIP, "%s: %s", what, hipGetErrorString(e));
  return TP_OK;
}

int run(const Spec &s, const Ptrs &q, int dt, void *ws, hipStream_t st, const char *what) {
  return run_planned(s, plan(s, dt), q, dt, ws, st, what);
}

// Two independent products of one pass.  In bf16 they share one launch when
// both plans fit the paired kernels: the first (long-K) product may be split
// along K, the second is not.  With `swapped` the second product's blocks are
// dispatched first and neither is split (a weight gradient s1 whose K, the
// token count, is short beside the activation gradient s2).  Otherwise they
// run one after the other with their own plans.  Plans depend on the sizes
// alone, so the workspace queries see the same ones.
struct PairPlan {
  bool paired = false, swapped = false;
  Plan p1, p2;
};

enum PairMode { PAIR_AUTO, PAIR_OFF, PAIR_SWAP };

PairPlan pair_plan_mode(const Spec &s1, const Spec &s2, int dt, PairMode mode) {
  PairPlan r;
  if (dt != TP_DT_BF16) {
    r.p1 = plan(s1, dt);
    r.p2 = plan(s2, dt);
    return r;
  }
  // apart: each with its own best plan
  r.p1 = plan_bf16(s1);
  r.p2 = plan_bf16(s2);
  double best = plan_us(s1, r.p1) + plan_us(s2, r.p2);
  if (mode == PAIR_OFF) return r;
  const bool force_swap = mode == PAIR_SWAP;
  if (force_swap) best = 1e30;
  // together: every built pair of variants with one residency, the first
  // possibly split along K
  Spec b = s2;
  b.can_split = false;
  std::vector<Plan> c2;
  for_each_plan(b, [&](const Plan &p) { c2.push_back(p); });
  GemmDesc d1, d2;
  std::memset(&d1, 0, sizeof d1);
  std::memset(&d2, 0, sizeof d2);
  d1.kseg = s1.kseg;
  d2.kseg = s2.kseg;
  for_each_plan(s1, [&](const Plan &p1) {
    for (const Plan &p2 : c2) {
      if (!p1.vec || !p2.vec || p1.res != p2.res) continue;
      if (tp_launch_gemm_pair(d1, variant(s1, p1), d2, variant(b, p2), nullptr, true, nullptr) != hipSuccess)
        continue;
      const int64_t n1 = plan_blocks(p1), n2 = plan_blocks(p2);
      const double t = kLaunchUs +
                       std::max(tile_cost(p1.bm, p1.bn, p1.res).first, tile_cost(p2.bm, p2.bn, p2.res).first) +
                       list_makespan(n1, block_us(s1, p1, n1 + n2), n2, block_us(b, p2, n1 + n2), plan_slots(p1)) +
                       reduce_us(s1, p1);
      if (t < best * 0.999 && !force_swap) {
        best = t;
        r.paired = true;
        r.p1 = p1;
        r.p2 = p2;
      }
    }
  });
  // swapped: s2's blocks first, neither split
  Spec f = s2, a = s1;
  f.can_split = false;
  a.can_split = false;
  std::vector<Plan> ca;
  for_each_plan(a, [&](const Plan &p) { ca.push_back(p); });
  for_each_plan(f, [&](const Plan &p2) {
    for (const Plan &p1 : ca) {
      if (!p1.vec || !p2.vec || p1.res != p2.res) continue;
      if (tp_launch_gemm_pair(d2, variant(f, p2), d1, variant(a, p1), nullptr, true, nullptr) != hipSuccess) continue;
      const int64_t n1 = plan_blocks(p1), n2 = plan_blocks(p2);
      const double t = kLaunchUs +
                       std::max(tile_cost(p1.bm, p1.bn, p1.res).first, tile_cost(p2.bm, p2.bn, p2.res).first) +
                       list_makespan(n2, block_us(f, p2, n1 + n2), n1, block_us(a, p1, n1 + n2), plan_slots(p2));
      if (t < best * 0.999) {
        best = t;
        r.paired = r.swapped = true;
        r.p1 = p1;
        r.p2 = p2;
      }
    }
  });
  return r;
}

// TP_GEMM_PAIR=off: always apart (timing comparisons; the parity tests use it
// to reach the single-launch paths of products that are normally paired);
// TP_GEMM_PAIR=swap: the swapped order whenever a pair of variants is built for
// it, else the usual choice (the parity tests reach its kernels at small sizes)
PairPlan pair_plan(const Spec &s1, const Spec &s2, int dt) {
  const char *env = std::getenv("TP_GEMM_PAIR");
  if (env != nullptr && std::strcmp(env, "off") == 0) return pair_plan_mode(s1, s2, dt, PAIR_OFF);
  if (env != nullptr && std::strcmp(env, "swap") == 0 && dt == TP_DT_BF16) {
    const PairPlan r = pair_plan_mode(s1, s2, dt, PAIR_SWAP);
    if (r.swapped) return r;
  }
  return pair_plan_mode(s1, s2, dt, PAIR_AUTO);
}

size_t pair_ws_bytes(const Spec &s1, const Spec &s2, int dt) {
  const PairPlan pp = pair_plan(s1, s2, dt);
  return std::max(align256(pp.p1.ws_bytes), align256(pp.p2.ws_bytes));
}

// A split-K reduction left for the next paired launch of the same call to run
// in extra workgroups (it must not write the partials this one reads).
struct PendingReduce {
  bool on = false;
  GemmDesc d;
};

// Run two independent products (paired when planned so).  `in` (may be null):
// a pending reduction of an earlier pair, run here first (inside the pair
// launch when there is one).  `out` (may be null): receives this pair's own
// split-K reduction instead of launching it, when it can run inside a later
// pair (bf16 output, 16-byte runs).
int run_pair(const Spec &s1, const Ptrs &q1, const Spec &s2, const Ptrs &q2, int dt, void *ws, hipStream_t st,
             const char *what1, const char *what2, PendingReduce *in = nullptr, PendingReduce *out = nullptr) {
  const PairPlan pp = pair_plan(s1, s2, dt);
  const GemmDesc *red = (in != nullptr && in->on) ? &in->d : nullptr;
  if (!pp.paired) {
    if (red != nullptr) {
      if (hipError_t e = tp_launch_splitk_reduce(*red, false, true, st))
        return fail(TP_EHIP, "%s: pending reduction: %s", what1, hipGetErrorString(e));
      in->on = false;
    }
    if (int e = run_planned(s1, pp.p1, q1, dt, ws, st, what1)) return e;
    return run_planned(s2, pp.p2, q2, dt, ws, st, what2);
  }
  if (pp.p1.splits > 1 && ws == nullptr) return fail(TP_EWORKSPACE, "%s: split-K plan without workspace", what1);
  log_plan(what1, s1, pp.p1, pp.swapped ? " (paired, second)" : " (paired, first)");
  log_plan(what2, s2, pp.p2, pp.swapped ? " (paired, first)" : " (paired, second)");
  const GemmDesc d1 = make_desc(s1, q1, pp.p1, dt, ws);
  const GemmDesc d2 = make_desc(s2, q2, pp.p2, dt, nullptr);
  hipError_t e = pp.swapped ? tp_launch_gemm_pair(d2, variant(s2, pp.p2), d1, variant(s1, pp.p1), red, false, st)
                            : tp_launch_gemm_pair(d1, variant(s1, pp.p1), d2, variant(s2, pp.p2), red, false, st);
  if (red != nullptr) in->on = false;
  if (e == hipSuccess && pp.p1.splits > 1) {
    if (out != nullptr && !s1.out_f32 && pp.p1.vec) {
      out->on = true;
      out->d = d1;
    } else {
      e = tp_launch_splitk_reduce(d1, s1.out_f32, pp.p1.vec, st);
    }
  }
  if (e != hipSuccess) return fail(TP_EHIP, "%s + %s: %s", what1, what2, hipGetErrorString(e));
  return TP_OK;
}

size_t esize(int dt) { return dt == TP_DT_F32 ? 4 : 2; }

// ---------------------------------------------------------------- specs
// MLP (all sizes already validated)
Spec spec_nn(int64_t M, int64_t N, int64_t K, int epi) {
  Spec s;
  s.layout = GEMM_NN;
  s.epi = epi;
  s.M = M;
  s.K = K;
  s.N = N;
  s.seg[0] = N;
  s.ld(K);   // A [M][K]
  s.ld(N);   // B [K][N], C [M][N]
  return s;
}
Spec spec_nt(int64_t M, int64_t N, int64_t K, int epi) {
  Spec s = spec_nn(M, N, K, epi);
  s.layout = GEMM_NT;
  return s;
}
Spec spec_tn(int64_t M, int64_t N, int64_t K) {
  Spec s;
  s.layout = GEMM_TN;
  s.epi = EPI_STORE;
  s.M = M;
  s.K = K;
  s.N = N;
  s.seg[0] = N;
  s.ld(M);   // A [K][M]
  s.ld(N);   // B [K][N], C [M][N]
  return s;
}

// tp_mlp_bwd workspace: dZ [s,ft] then the split-K partials of dW1 / dW2
struct MlpBwdLayout {
  Spec g_dz, g_dw2, g_dx, g_dw1;
  size_t dz_bytes = 0, part1_bytes = 0, part2_bytes = 0, total = 0;
};
MlpBwdLayout mlp_bwd_layout(int dt, int64_t s, int64_t h, int64_t ft) {
  MlpBwdLayout L;
  L.g_dz = spec_nt(s, ft, h, EPI_ACT_BWD);
  L.g_dz.ld(h);
  L.g_dw2 = spec_tn(ft, h, s);
  L.g_dx = spec_nt(s, h, ft, EPI_STORE);
  L.g_dw1 = spec_tn(h, ft, s);
  for (Spec *g : {&L.g_dz, &L.g_dw2, &L.g_dx, &L.g_dw1}) g->can_split = true;
  L.dz_bytes = align256((size_t)s * ft * esize(dt));
  // the two passes' split-K partials apart: the second pass runs the first's reduction
  L.part1_bytes = align256(pair_ws_bytes(L.g_dw2, L.g_dz, dt));
  L.part2_bytes = align256(pair_ws_bytes(L.g_dw1, L.g_dx, dt));
  L.total = L.dz_bytes + L.part1_bytes + L.part2_bytes;
  return L;
}

struct SwigluBwdLayout {
  Spec g_da, g_dwd, g_dx, g_dwgu;
  size_t dg_bytes = 0, part1_bytes = 0, part2_bytes = 0, total = 0;
};
SwigluBwdLayout swiglu_bwd_layout(int dt, int64_t s, int64_t h, int64_t ft) {
  SwigluBwdLayout L;
  L.g_da = spec_nt(s, ft, h, EPI_SWIGLU_BWD);
  L.g_dwd = spec_tn(ft, h, s);
  // dX = dG.Wg^T + dU.Wu^T: two K-segments of width ft
  Spec dx;
  dx.layout = GEMM_NT;
  dx.epi = EPI_STORE;
  dx.M = s;
  dx.N = h;
  dx.K = 2 * ft;
  dx.nseg = 2;
  dx.kseg = true;
  dx.seg[0] = dx.seg[1] = ft;
  dx.ld(ft);
  dx.ld(h);
  L.g_dx = dx;
  // [dWg | dWu] = X^T . [dG | dU]: two N-segments of width ft
  Spec dw;
  dw.layout = GEMM_TN;
  dw.epi = EPI_STORE;
  dw.M = h;
  dw.K = s;
  dw.nseg = 2;
  dw.seg[0] = dw.seg[1] = ft;
  dw.N = 2 * ft;
  dw.ld(h);
  dw.ld(ft);
  L.g_dwgu = dw;
  for (Spec *g : {&L.g_da, &L.g_dwd, &L.g_dx, &L.g_dwgu}) g->can_split = true;
  L.dg_bytes = align256((size_t)s * ft * esize(dt));
  L.part1_bytes = align256(pair_ws_bytes(L.g_dwd, L.g_da, dt));
  L.part2_bytes = align256(pair_ws_bytes(L.g_dwgu, L.g_dx, dt));
  L.total = 2 * L.dg_bytes + L.part1_bytes + L.part2_bytes;
  return L;
}

struct AttnBwdLayout {
  Spec g_dx, g_dwqkv, g_do, g_dwo;
  size_t part1_bytes = 0, part2_bytes = 0, total = 0;
};
AttnBwdLayout attn_bwd_layout(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv) {
  AttnBwdLayout L;
  Spec dx;
  dx.layout = GEMM_NT;
  dx.epi = EPI_STORE;
  dx.M = s;
  dx.N = h;
  dx.K = dq + 2 * dkv;
  dx.nseg = 3;
  dx.kseg = true;
  dx.seg[0] = dq;
  dx.seg[1] = dx.seg[2] = dkv;
  dx.ld(dq);
  dx.ld(dkv);
  dx.ld(h);
  L.g_dx = dx;
  Spec dw;
  dw.layout = GEMM_TN;
  dw.epi = EPI_STORE;
  dw.M = h;
  dw.K = s;
  dw.nseg = 3;
  dw.seg[0] = dq;
  dw.seg[1] = dw.seg[2] = dkv;
  dw.N = dq + 2 * dkv;
  dw.ld(h);
  dw.ld(dq);
  dw.ld(dkv);
  L.g_dwqkv = dw;
  L.g_do = spec_nt(s, dq, h, EPI_STORE);
  L.g_dwo = spec_tn(dq, h, s);
  for (Spec *g : {&L.g_dx, &L.g_dwqkv, &L.g_do, &L.g_dwo}) g->can_split = true;
  L.part1_bytes = align256(pair_ws_bytes(L.g_dwqkv, L.g_dx, dt));
  L.part2_bytes = align256(pair_ws_bytes(L.g_dwo, L.g_do, dt));
  L.total = L.part1_bytes + L.part2_bytes;
  return L;
}

// fused LM head + CE statistics: the GEMM's plan and its partial-statistics workspace
struct LmCePlan {
  Spec g;
  Plan p;
  int parts = 0;
  size_t bytes = 0;
};
LmCePlan lm_ce_plan(int64_t s, int64_t h, int64_t Vs) {
  LmCePlan L;
  L.g = spec_nn(s, Vs, h, EPI_CE_STATS);
  L.g.out_f32 = true;
  L.p = plan_bf16(L.g);
  L.parts = L.p.tiles_n;  // one part per tile column: max [parts][s], sum exp [parts][s], target logit [s]
  L.bytes = align256((size_t)s * (2 * (size_t)L.parts + 1) * sizeof(float));
  return L;
}

bool ws_ok(Checker &c, const void *ws, size_t have, size_t need, const char *call) {
  if (c.status) return false;
  if (need == 0) return true;
  if (ws == nullptr || have < need) {
    c.status = fail(TP_EWORKSPACE, "%s needs %zu workspace bytes, got %zu (%p)", call, need, have, ws);
    return false;
  }
  if (((uintptr_t)ws & 255) != 0) {
    c.status = fail(TP_EALIGN, "%s: workspace %p is not 256-byte aligned", call, ws);
    return false;
  }
  return true;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char *tp_status_string(int status) {
  switch (status) {
  case TP_OK: return "TP_OK";
  case TP_EINVAL: return "TP_EINVAL";
  case TP_ESHAPE: return "TP_ESHAPE";
  case TP_EDTYPE: return "TP_EDTYPE";
  case TP_EALIGN: return "TP_EALIGN";
  case TP_EWORKSPACE: return "TP_EWORKSPACE";
  case TP_EHIP: return "TP_EHIP";
  case TP_EUNSUPPORTED: return "TP_EUNSUPPORTED";
  }
  return "TP_UNKNOWN_STATUS";
}

const char *tp_last_error(void) { return g_last_error.c_str(); }

int tp_abi_version(void) { return TP_ABI_VERSION; }

// ------------------------------------------------------------------ MLP
int tp_mlp_fwd(int act, int dt, int64_t s, int64_t h, int64_t ft, const void *X, const void *W1,
               const void *W2, void *Z, void *H, void *Y, void *stream) {
  Checker c;
  int64_t nx, nw, nz;
  c.act(act);
  c.dtype(dt, true, "tp_mlp_fwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  c.elems(s, h, nx, "X") && c.elems(h, ft, nw, "W1") && c.elems(s, ft, nz, "Z");
  c.ptr(X, nx, "X") && c.ptr(W1, nw, "W1") && c.ptr(W2, nw, "W2") && c.ptr(H, nz, "H") && c.ptr(Y, nx, "Y");
  if (!c.status && act == TP_ACT_GELU) c.ptr(Z, nz, "Z");
  if (!c.status && Z) c.ptr(Z, nz, "Z");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  Spec g1 = spec_nn(s, ft, h, EPI_ACT_FWD);
  Ptrs p1;
  p1.A[0] = X; p1.lda[0] = h;
  p1.B[0] = W1; p1.ldb[0] = ft;
  p1.C[0] = H; p1.ldc[0] = ft;
  p1.ao0 = Z; p1.ldao = ft;
  p1.act = act == TP_ACT_GELU ? ACT_GELU : ACT_RELU;
  p1.stream_out = 1 | 2;
  if (int e = run(g1, p1, dt, nullptr, st, "tp_mlp_fwd column GEMM")) return e;
  Spec g2 = spec_nn(s, h, ft, EPI_STORE);
  Ptrs p2;
  p2.A[0] = H; p2.lda[0] = ft;
  p2.B[0] = W2; p2.ldb[0] = h;
  p2.C[0] = Y; p2.ldc[0] = h;
  p2.stream_out = 1;
  if (int e = run(g2, p2, dt, nullptr, st, "tp_mlp_fwd row GEMM")) return e;
  return ok();
}

size_t tp_mlp_bwd_workspace(int dt, int64_t s, int64_t h, int64_t ft) {
  Checker c;
  c.dtype(dt, true, "tp_mlp_bwd_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  if (c.status) return 0;
  return mlp_bwd_layout(dt, s, h, ft).total;
}

int tp_mlp_bwd(int act, int dt, int64_t s, int64_t h, int64_t ft, const void *X, const void *W1,
               const void *W2, const void *Z, const void *H, const void *dY, void *dX, void *dW1,
               void *dW2, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nx, nw, nz;
  c.act(act);
  c.dtype(dt, true, "tp_mlp_bwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  c.elems(s, h, nx, "X") && c.elems(h, ft, nw, "W1") && c.elems(s, ft, nz, "Z");
  c.ptr(X, nx, "X") && c.ptr(W1, nw, "W1") && c.ptr(W2, nw, "W2") && c.ptr(H, nz, "H") &&
      c.ptr(dY, nx, "dY") && c.ptr(dX, nx, "dX") && c.ptr(dW1, nw, "dW1") && c.ptr(dW2, nw, "dW2");
  if (!c.status && act == TP_ACT_GELU) c.ptr(Z, nz, "Z");
  if (!c.status && Z) c.ptr(Z, nz, "Z");
  if (c.status) return c.status;
  const MlpBwdLayout L = mlp_bwd_layout(dt, s, h, ft);
  ws_ok(c, ws, ws_bytes, L.total, "tp_mlp_bwd");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  char *wsb = (char *)ws;
  void *dZ = wsb;
  void *part1 = wsb + L.dz_bytes, *part2 = wsb + L.dz_bytes + L.part1_bytes;
  PendingReduce pend;
  const int a = act == TP_ACT_GELU ? ACT_GELU : ACT_RELU;
  {  // dW2 = H^T . dY  beside  dZ = (dY . W2^T) * act'(Z)  (ReLU mask from Z, or from H without Z)
    Ptrs pw;
    pw.A[0] = H; pw.lda[0] = ft;
    pw.B[0] = dY; pw.ldb[0] = h;
    pw.C[0] = dW2; pw.ldc[0] = h;
    Ptrs pz;
    pz.A[0] = dY; pz.lda[0] = h;
    pz.B[0] = W2; pz.ldb[0] = h;
    pz.C[0] = dZ; pz.ldc[0] = ft;
    pz.ai0 = Z ? Z : H; pz.ldai = ft;
    pz.act = a;
    if (int e = run_pair(L.g_dw2, pw, L.g_dz, pz, dt, part1, st, "tp_mlp_bwd dW2 GEMM", "tp_mlp_bwd dZ GEMM",
                         nullptr, &pend))
      return e;
  }
  {  // dW1 = X^T . dZ  beside  dX = dZ . W1^T
    Ptrs pw;
    pw.A[0] = X; pw.lda[0] = h;
    pw.B[0] = dZ; pw.ldb[0] = ft;
    pw.C[0] = dW1; pw.ldc[0] = ft;
    Ptrs px;
    px.A[0] = dZ; px.lda[0] = ft;
    px.B[0] = W1; px.ldb[0] = ft;
    px.C[0] = dX; px.ldc[0] = h;
    if (int e = run_pair(L.g_dw1, pw, L.g_dx, px, dt, part2, st, "tp_mlp_bwd dW1 GEMM", "tp_mlp_bwd dX GEMM",
                         &pend))
      return e;
  }
  return ok();
}

// ------------------------------------------------------------------ SwiGLU
int tp_swiglu_fwd(int dt, int64_t s, int64_t h, int64_t ft, const void *X, const void *Wg, const void *Wu,
                  const void *Wd, void *G, void *U, void *A, void *Y, void *stream) {
  Checker c;
  int64_t nx, nw, nz;
  c.dtype(dt, true, "tp_swiglu_fwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  c.elems(s, h, nx, "X") && c.elems(h, ft, nw, "Wg") && c.elems(s, ft, nz, "G");
  c.ptr(X, nx, "X") && c.ptr(Wg, nw, "Wg") && c.ptr(Wu, nw, "Wu") && c.ptr(Wd, nw, "Wd") &&
      c.ptr(G, nz, "G") && c.ptr(U, nz, "U") && c.ptr(A, nz, "A") && c.ptr(Y, nx, "Y");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  {  // G = X.Wg, U = X.Wu (one dual-B pass), A = SiLU(G) * U
    Spec g = spec_nn(s, ft, h, EPI_SWIGLU_FWD);
    g.dual = true;
    Ptrs p;
    p.A[0] = X; p.lda[0] = h;
    p.B[0] = Wg; p.B[1] = Wu; p.ldb[0] = p.ldb[1] = ft;
    p.C[0] = A; p.ldc[0] = ft;
    p.ao0 = G; p.ao1 = U; p.ldao = ft;
    if (int e = run(g, p, dt, nullptr, st, "tp_swiglu_fwd gate/up GEMM")) return e;
  }
  {  // Y = A . Wd
    Spec g = spec_nn(s, h, ft, EPI_STORE);
    Ptrs p;
    p.A[0] = A; p.lda[0] = ft;
    p.B[0] = Wd; p.ldb[0] = h;
    p.C[0] = Y; p.ldc[0] = h;
    p.stream_out = 1;
    if (int e = run(g, p, dt, nullptr, st, "tp_swiglu_fwd down GEMM")) return e;
  }
  return ok();
}

size_t tp_swiglu_bwd_workspace(int dt, int64_t s, int64_t h, int64_t ft) {
  Checker c;
  c.dtype(dt, true, "tp_swiglu_bwd_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  if (c.status) return 0;
  return swiglu_bwd_layout(dt, s, h, ft).total;
}

int tp_swiglu_bwd(int dt, int64_t s, int64_t h, int64_t ft, const void *X, const void *Wg, const void *Wu,
                  const void *Wd, const void *G, const void *U, const void *A, const void *dY, void *dX,
                  void *dWg, void *dWu, void *dWd, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nx, nw, nz;
  c.dtype(dt, true, "tp_swiglu_bwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(ft, "ft");
  c.elems(s, h, nx, "X") && c.elems(h, ft, nw, "Wg") && c.elems(s, ft, nz, "G");
  c.ptr(X, nx, "X") && c.ptr(Wg, nw, "Wg") && c.ptr(Wu, nw, "Wu") && c.ptr(Wd, nw, "Wd") &&
      c.ptr(G, nz, "G") && c.ptr(U, nz, "U") && c.ptr(A, nz, "A") && c.ptr(dY, nx, "dY") &&
      c.ptr(dX, nx, "dX") && c.ptr(dWg, nw, "dWg") && c.ptr(dWu, nw, "dWu") && c.ptr(dWd, nw, "dWd");
  if (c.status) return c.status;
  const SwigluBwdLayout L = swiglu_bwd_layout(dt, s, h, ft);
  ws_ok(c, ws, ws_bytes, L.total, "tp_swiglu_bwd");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  char *wsb = (char *)ws;
  void *dG = wsb, *dU = wsb + L.dg_bytes, *part1 = wsb + 2 * L.dg_bytes;
  void *part2 = (char *)part1 + L.part1_bytes;
  PendingReduce pend;
  {  // dWd = A^T . dY  beside  dA = dY . Wd^T, dG = dA * U * SiLU'(G), dU = dA * SiLU(G)
    Ptrs pw;
    pw.A[0] = A; pw.lda[0] = ft;
    pw.B[0] = dY; pw.ldb[0] = h;
    pw.C[0] = dWd; pw.ldc[0] = h;
    Ptrs pa;
    pa.A[0] = dY; pa.lda[0] = h;
    pa.B[0] = Wd; pa.ldb[0] = h;
    pa.C[0] = dG; pa.ldc[0] = ft;
    pa.ai0 = G; pa.ai1 = U; pa.ldai = ft;
    pa.ao0 = dU; pa.ldao = ft;
    pw.stream_out = 1;
    pa.stream_out = 1 | 2;
    if (int e = run_pair(L.g_dwd, pw, L.g_da, pa, dt, part1, st, "tp_swiglu_bwd dWd GEMM", "tp_swiglu_bwd dA GEMM",
                         nullptr, &pend))
      return e;
  }
  {  // [dWg | dWu] = X^T . [dG | dU]  beside  dX = dG . Wg^T + dU . Wu^T
    Ptrs pw;
    pw.A[0] = X; pw.lda[0] = h;
    pw.B[0] = dG; pw.B[1] = dU; pw.ldb[0] = pw.ldb[1] = ft;
    pw.C[0] = dWg; pw.C[1] = dWu; pw.ldc[0] = pw.ldc[1] = ft;
    Ptrs px;
    px.A[0] = dG; px.A[1] = dU; px.lda[0] = px.lda[1] = ft;
    px.B[0] = Wg; px.B[1] = Wu; px.ldb[0] = px.ldb[1] = ft;
    px.C[0] = dX; px.ldc[0] = h;
    pw.stream_out = px.stream_out = 1;
    if (int e = run_pair(L.g_dwgu, pw, L.g_dx, px, dt, part2, st, "tp_swiglu_bwd dWg/dWu GEMM",
                         "tp_swiglu_bwd dX GEMM", &pend))
      return e;
  }
  return ok();
}

// ------------------------------------------------------------------ attention projections
int tp_attn_proj_fwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv, const void *X, const void *Wq,
                     const void *Wk, const void *Wv, const void *O, const void *Wo, void *Q, void *K, void *V,
                     void *Y, void *stream) {
  Checker c;
  int64_t nx, nwq, nwk, nq, nk;
  c.dtype(dt, true, "tp_attn_proj_fwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq") && c.dim(dkv, "dkv");
  c.elems(s, h, nx, "X") && c.elems(h, dq, nwq, "Wq") && c.elems(h, dkv, nwk, "Wk") &&
      c.elems(s, dq, nq, "Q") && c.elems(s, dkv, nk, "K");
  c.ptr(X, nx, "X") && c.ptr(Wq, nwq, "Wq") && c.ptr(Wk, nwk, "Wk") && c.ptr(Wv, nwk, "Wv") &&
      c.ptr(O, nq, "O") && c.ptr(Wo, nwq, "Wo") && c.ptr(Q, nq, "Q") && c.ptr(K, nk, "K") &&
      c.ptr(V, nk, "V") && c.ptr(Y, nx, "Y");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  // [Q | K | V] = X . [Wq | Wk | Wv] (three N-segments)  beside  Y = O . Wo
  Spec gq;
  gq.layout = GEMM_NN;
  gq.epi = EPI_STORE;
  gq.M = s;
  gq.K = h;
  gq.nseg = 3;
  gq.seg[0] = dq;
  gq.seg[1] = gq.seg[2] = dkv;
  gq.N = dq + 2 * dkv;
  gq.ld(h);
  gq.ld(dq);
  gq.ld(dkv);
  Ptrs pq;
  pq.A[0] = X; pq.lda[0] = h;
  pq.B[0] = Wq; pq.B[1] = Wk; pq.B[2] = Wv;
  pq.ldb[0] = dq; pq.ldb[1] = pq.ldb[2] = dkv;
  pq.C[0] = Q; pq.C[1] = K; pq.C[2] = V;
  pq.ldc[0] = dq; pq.ldc[1] = pq.ldc[2] = dkv;
  const Spec go = spec_nn(s, h, dq, EPI_STORE);
  Ptrs po;
  po.A[0] = O; po.lda[0] = dq;
  po.B[0] = Wo; po.ldb[0] = h;
  po.C[0] = Y; po.ldc[0] = h;
  pq.stream_out = po.stream_out = 1;
  if (int e = run_pair(gq, pq, go, po, dt, nullptr, st, "tp_attn_proj_fwd QKV GEMM", "tp_attn_proj_fwd output GEMM"))
    return e;
  return ok();
}

size_t tp_attn_proj_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv) {
  Checker c;
  c.dtype(dt, true, "tp_attn_proj_bwd_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq") && c.dim(dkv, "dkv");
  if (c.status) return 0;
  return attn_bwd_layout(dt, s, h, dq, dkv).total;
}

int tp_attn_proj_bwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv, const void *X, const void *Wq,
                     const void *Wk, const void *Wv, const void *O, const void *Wo, const void *dQ,
                     const void *dK, const void *dV, const void *dY, void *dX, void *dWq, void *dWk,
                     void *dWv, void *dO, void *dWo, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nx, nwq, nwk, nq, nk;
  c.dtype(dt, true, "tp_attn_proj_bwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq") && c.dim(dkv, "dkv");
  c.elems(s, h, nx, "X") && c.elems(h, dq, nwq, "Wq") && c.elems(h, dkv, nwk, "Wk") &&
      c.elems(s, dq, nq, "Q") && c.elems(s, dkv, nk, "K");
  c.ptr(X, nx, "X") && c.ptr(Wq, nwq, "Wq") && c.ptr(Wk, nwk, "Wk") && c.ptr(Wv, nwk, "Wv") &&
      c.ptr(O, nq, "O") && c.ptr(Wo, nwq, "Wo") && c.ptr(dQ, nq, "dQ") && c.ptr(dK, nk, "dK") &&
      c.ptr(dV, nk, "dV") && c.ptr(dY, nx, "dY") && c.ptr(dX, nx, "dX") && c.ptr(dWq, nwq, "dWq") &&
      c.ptr(dWk, nwk, "dWk") && c.ptr(dWv, nwk, "dWv") && c.ptr(dO, nq, "dO") && c.ptr(dWo, nwq, "dWo");
  if (c.status) return c.status;
  const AttnBwdLayout L = attn_bwd_layout(dt, s, h, dq, dkv);
  ws_ok(c, ws, ws_bytes, L.total, "tp_attn_proj_bwd");
  if (c.status) return c.status;
  hipStream_t st = (hipStream_t)stream;
  void *part1 = ws, *part2 = (char *)ws + L.part1_bytes;
  PendingReduce pend;
  {  // [dWq | dWk | dWv] = X^T . [dQ | dK | dV]  beside  dX = dQ.Wq^T + dK.Wk^T + dV.Wv^T (K-segments)
    Ptrs pw;
    pw.A[0] = X; pw.lda[0] = h;
    pw.B[0] = dQ; pw.B[1] = dK; pw.B[2] = dV;
    pw.ldb[0] = dq; pw.ldb[1] = pw.ldb[2] = dkv;
    pw.C[0] = dWq; pw.C[1] = dWk; pw.C[2] = dWv;
    pw.ldc[0] = dq; pw.ldc[1] = pw.ldc[2] = dkv;
    Ptrs px;
    px.A[0] = dQ; px.A[1] = dK; px.A[2] = dV;
    px.lda[0] = dq; px.lda[1] = px.lda[2] = dkv;
    px.B[0] = Wq; px.B[1] = Wk; px.B[2] = Wv;
    px.ldb[0] = dq; px.ldb[1] = px.ldb[2] = dkv;
    px.C[0] = dX; px.ldc[0] = h;
    pw.stream_out = px.stream_out = 1;
    if (int e = run_pair(L.g_dwqkv, pw, L.g_dx, px, dt, part1, st, "tp_attn_proj_bwd dWqkv GEMM",
                         "tp_attn_proj_bwd dX GEMM", nullptr, &pend))
      return e;
  }
  {  // dWo = O^T . dY  beside  dO = dY . Wo^T
    Ptrs pw;
    pw.A[0] = O; pw.lda[0] = dq;
    pw.B[0] = dY; pw.ldb[0] = h;
    pw.C[0] = dWo; pw.ldc[0] = h;
    Ptrs po;
    po.A[0] = dY; po.lda[0] = h;
    po.B[0] = Wo; po.ldb[0] = h;
    po.C[0] = dO; po.ldc[0] = dq;
    pw.stream_out = po.stream_out = 1;
    if (int e = run_pair(L.g_dwo, pw, L.g_do, po, dt, part2, st, "tp_attn_proj_bwd dWo GEMM",
                         "tp_attn_proj_bwd dO GEMM", &pend))
      return e;
  }
  return ok();
}

// The two halves of tp_attn_proj_bwd as calls of their own, for a layer
// backward that runs the attention core's backward between them: the output
// projection's (dO, dWo) first, then the Q/K/V projections' (dX, dWq/k/v).
size_t tp_attn_out_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq) {
  Checker c;
  c.dtype(dt, true, "tp_attn_out_bwd_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq");
  if (c.status) return 0;
  const AttnBwdLayout L = attn_bwd_layout(dt, s, h, dq, 0);
  return L.part2_bytes;
}

int tp_attn_out_bwd(int dt, int64_t s, int64_t h, int64_t dq, const void *O, const void *Wo, const void *dY,
                    void *dO, void *dWo, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nx, nwq, nq;
  c.dtype(dt, true, "tp_attn_out_bwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq");
  c.elems(s, h, nx, "dY") && c.elems(h, dq, nwq, "Wo") && c.elems(s, dq, nq, "O");
  c.ptr(O, nq, "O") && c.ptr(Wo, nwq, "Wo") && c.ptr(dY, nx, "dY") && c.ptr(dO, nq, "dO") && c.ptr(dWo, nwq, "dWo");
  if (c.status) return c.status;
  const AttnBwdLayout L = attn_bwd_layout(dt, s, h, dq, 0);
  ws_ok(c, ws, ws_bytes, L.part2_bytes, "tp_attn_out_bwd");
  if (c.status) return c.status;
  Ptrs pw;
  pw.A[0] = O; pw.lda[0] = dq;
  pw.B[0] = dY; pw.ldb[0] = h;
  pw.C[0] = dWo; pw.ldc[0] = h;
  Ptrs po;
  po.A[0] = dY; po.lda[0] = h;
  po.B[0] = Wo; po.ldb[0] = h;
  po.C[0] = dO; po.ldc[0] = dq;
  pw.stream_out = po.stream_out = 1;
  if (int e = run_pair(L.g_dwo, pw, L.g_do, po, dt, ws, (hipStream_t)stream, "tp_attn_out_bwd dWo GEMM",
                       "tp_attn_out_bwd dO GEMM"))
    return e;
  return ok();
}

size_t tp_attn_qkv_bwd_workspace(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv) {
  Checker c;
  c.dtype(dt, true, "tp_attn_qkv_bwd_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq") && c.dim(dkv, "dkv");
  if (c.status) return 0;
  return attn_bwd_layout(dt, s, h, dq, dkv).part1_bytes;
}

int tp_attn_qkv_bwd(int dt, int64_t s, int64_t h, int64_t dq, int64_t dkv, const void *X, const void *Wq,
                    const void *Wk, const void *Wv, const void *dQ, const void *dK, const void *dV, void *dX,
                    void *dWq, void *dWk, void *dWv, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nx, nwq, nwk, nq, nk;
  c.dtype(dt, true, "tp_attn_qkv_bwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(dq, "dq") && c.dim(dkv, "dkv");
  c.elems(s, h, nx, "X") && c.elems(h, dq, nwq, "Wq") && c.elems(h, dkv, nwk, "Wk") &&
      c.elems(s, dq, nq, "dQ") && c.elems(s, dkv, nk, "dK");
  c.ptr(X, nx, "X") && c.ptr(Wq, nwq, "Wq") && c.ptr(Wk, nwk, "Wk") && c.ptr(Wv, nwk, "Wv") &&
      c.ptr(dQ, nq, "dQ") && c.ptr(dK, nk, "dK") && c.ptr(dV, nk, "dV") && c.ptr(dX, nx, "dX") &&
      c.ptr(dWq, nwq, "dWq") && c.ptr(dWk, nwk, "dWk") && c.ptr(dWv, nwk, "dWv");
  if (c.status) return c.status;
  const AttnBwdLayout L = attn_bwd_layout(dt, s, h, dq, dkv);
  ws_ok(c, ws, ws_bytes, L.part1_bytes, "tp_attn_qkv_bwd");
  if (c.status) return c.status;
  Ptrs pw;
  pw.A[0] = X; pw.lda[0] = h;
  pw.B[0] = dQ; pw.B[1] = dK; pw.B[2] = dV;
  pw.ldb[0] = dq; pw.ldb[1] = pw.ldb[2] = dkv;
  pw.C[0] = dWq; pw.C[1] = dWk; pw.C[2] = dWv;
  pw.ldc[0] = dq; pw.ldc[1] = pw.ldc[2] = dkv;
  Ptrs px;
  px.A[0] = dQ; px.A[1] = dK; px.A[2] = dV;
  px.lda[0] = dq; px.lda[1] = px.lda[2] = dkv;
  px.B[0] = Wq; px.B[1] = Wk; px.B[2] = Wv;
  px.ldb[0] = dq; px.ldb[1] = px.ldb[2] = dkv;
  px.C[0] = dX; px.ldc[0] = h;
  pw.stream_out = px.stream_out = 1;
  if (int e = run_pair(L.g_dwqkv, pw, L.g_dx, px, dt, ws, (hipStream_t)stream, "tp_attn_qkv_bwd dWqkv GEMM",
                       "tp_attn_qkv_bwd dX GEMM"))
    return e;
  return ok();
}

// ------------------------------------------------------------------ vocab
int tp_lm_head_fwd(int dt, int64_t s, int64_t h, int64_t Vs, const void *Hf, const void *Wlm, float *logits,
                   void *stream) {
  Checker c;
  int64_t nh, nw, nl;
  c.dtype(dt, true, "tp_lm_head_fwd");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(Vs, "Vs");
  c.elems(s, h, nh, "Hf") && c.elems(h, Vs, nw, "Wlm") && c.elems(s, Vs, nl, "logits");
  c.ptr(Hf, nh, "Hf") && c.ptr(Wlm, nw, "Wlm") && c.ptr(logits, nl, "logits");
  if (c.status) return c.status;
  Spec g = spec_nn(s, Vs, h, EPI_STORE);
  g.out_f32 = true;
  Ptrs p;
  p.A[0] = Hf; p.lda[0] = h;
  p.B[0] = Wlm; p.ldb[0] = Vs;
  p.C[0] = logits; p.ldc[0] = Vs;
  if (int e = run(g, p, dt, nullptr, (hipStream_t)stream, "tp_lm_head_fwd GEMM")) return e;
  return ok();
}

int tp_vocab_ce(int64_t s, int64_t Vs, int64_t vocab_start, const float *logits, const int64_t *target,
                float *lmax, float *lsumexp, float *tlogit, void *stream) {
  Checker c;
  int64_t nl;
  c.dim(s, "s") && c.dim(Vs, "Vs");
  if (!c.status && vocab_start < 0) c.status = fail(TP_ESHAPE, "vocab_start = %lld < 0", (long long)vocab_start);
  c.elems(s, Vs, nl, "logits");
  c.ptr(logits, nl, "logits") && c.ptr(target, s, "target") && c.ptr(lmax, s, "lmax") &&
      c.ptr(lsumexp, s, "lsumexp") && c.ptr(tlogit, s, "tlogit");
  if (c.status) return c.status;
  hipError_t e = tp_launch_vocab_ce(s, Vs, vocab_start, logits, target, lmax, lsumexp, tlogit,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_vocab_ce: %s", hipGetErrorString(e));
  return ok();
}

int tp_vocab_ce_bwd(int dt, int64_t s, int64_t Vs, int64_t vocab_start, const float *logits,
                    const int64_t *target, const float *gmax, const float *gsum, const float *dloss,
                    void *dlogits, void *stream) {
  Checker c;
  int64_t nl;
  c.dtype(dt, true, "tp_vocab_ce_bwd");
  c.dim(s, "s") && c.dim(Vs, "Vs");
  if (!c.status && vocab_start < 0) c.status = fail(TP_ESHAPE, "vocab_start = %lld < 0", (long long)vocab_start);
  c.elems(s, Vs, nl, "logits");
  c.ptr(logits, nl, "logits") && c.ptr(target, s, "target") && c.ptr(gmax, s, "gmax") &&
      c.ptr(gsum, s, "gsum") && c.ptr(dloss, s, "dloss") && c.ptr(dlogits, nl, "dlogits");
  if (c.status) return c.status;
  hipError_t e = tp_launch_vocab_ce_bwd(dt == TP_DT_BF16, s, Vs, vocab_start, logits, target, gmax, gsum, dloss,
                                        dlogits, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_vocab_ce_bwd: %s", hipGetErrorString(e));
  return ok();
}

int tp_attn_core_fwd(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d, const void *Q, const void *K,
                     const void *V, void *O, float *lse, void *stream) {
  Checker c;
  int64_t nqe, nke, nl;
  c.dtype(dt, false, "tp_attn_core_fwd");
  c.dim(s, "s") && c.dim(nq, "nq") && c.dim(nkv, "nkv") && c.dim(d, "d");
  if (!c.status && d != 128) c.status = fail(TP_EUNSUPPORTED, "tp_attn_core_fwd: head dim %lld (only 128)", (long long)d);
  if (!c.status && nq > 0 && (nkv == 0 || nq % nkv != 0))
    c.status = fail(TP_ESHAPE, "tp_attn_core_fwd: nq = %lld is not a multiple of nkv = %lld", (long long)nq,
                    (long long)nkv);
  c.elems(s, nq * d, nqe, "Q") && c.elems(s, nkv * d, nke, "K") && c.elems(nq, s, nl, "lse");
  c.ptr(Q, nqe, "Q") && c.ptr(K, nke, "K") && c.ptr(V, nke, "V") && c.ptr(O, nqe, "O") && c.ptr(lse, nl, "lse");
  if (c.status) return c.status;
  hipError_t e = tp_launch_attn_fwd(s, nq, nkv, Q, K, V, O, lse, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_attn_core_fwd: %s", hipGetErrorString(e));
  return ok();
}

size_t tp_attn_core_bwd_workspace(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d) {
  Checker c;
  c.dtype(dt, false, "tp_attn_core_bwd_workspace");
  c.dim(s, "s") && c.dim(nq, "nq") && c.dim(nkv, "nkv") && c.dim(d, "d");
  if (!c.status && d != 128) return 0;
  if (c.status) return 0;
  return tp_attn_bwd_ws_bytes(s, nq);
}

int tp_attn_core_bwd(int dt, int64_t s, int64_t nq, int64_t nkv, int64_t d, const void *Q, const void *K,
                     const void *V, const void *O, const void *dO, const float *lse, void *dQ, void *dK, void *dV,
                     void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t nqe, nke, nl;
  c.dtype(dt, false, "tp_attn_core_bwd");
  c.dim(s, "s") && c.dim(nq, "nq") && c.dim(nkv, "nkv") && c.dim(d, "d");
  if (!c.status && d != 128) c.status = fail(TP_EUNSUPPORTED, "tp_attn_core_bwd: head dim %lld (only 128)", (long long)d);
  if (!c.status && (nq % (nkv ? nkv : 1) != 0 || (nkv == 0) != (nq == 0)))
    c.status = fail(TP_ESHAPE, "tp_attn_core_bwd: nq = %lld is not a positive multiple of nkv = %lld "
                    "(or both 0)", (long long)nq, (long long)nkv);
  c.elems(s, nq * d, nqe, "Q") && c.elems(s, nkv * d, nke, "K") && c.elems(nq, s, nl, "lse");
  c.ptr(Q, nqe, "Q") && c.ptr(K, nke, "K") && c.ptr(V, nke, "V") && c.ptr(O, nqe, "O") && c.ptr(dO, nqe, "dO") &&
      c.ptr(lse, nl, "lse") && c.ptr(dQ, nqe, "dQ") && c.ptr(dK, nke, "dK") && c.ptr(dV, nke, "dV");
  if (c.status) return c.status;
  ws_ok(c, ws, ws_bytes, nqe > 0 ? tp_attn_bwd_ws_bytes(s, nq) : 0, "tp_attn_core_bwd");
  if (c.status) return c.status;
  hipError_t e = tp_launch_attn_bwd(s, nq, nkv, Q, K, V, O, dO, lse, dQ, dK, dV, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_attn_core_bwd: %s", hipGetErrorString(e));
  return ok();
}

int tp_sp_ln_fwd(int dt, int64_t n, int64_t h, float p, float eps, const void *y, const void *x,
                 const uint8_t *mask, const void *gamma, const void *beta, void *u, void *z, float *mean,
                 float *rstd, void *stream) {
  Checker c;
  int64_t ne;
  c.dtype(dt, false, "tp_sp_ln_fwd");
  c.dim(n, "n") && c.dim(h, "h");
  if (!c.status && !(p >= 0.f && p < 1.f)) c.status = fail(TP_EINVAL, "tp_sp_ln_fwd: dropout p = %g not in [0, 1)", p);
  if (!c.status && !(eps > 0.f)) c.status = fail(TP_EINVAL, "tp_sp_ln_fwd: eps = %g is not positive", eps);
  if (!c.status && tp_sp_ln_passes(h) > 2) c.status = fail(TP_EUNSUPPORTED, "tp_sp_ln_fwd: h = %lld > 16384", (long long)h);
  c.elems(n, h, ne, "x");
  c.ptr(y, ne, "y") && c.ptr(x, ne, "x") && c.ptr(mask, ne, "mask") && c.ptr(gamma, h, "gamma") &&
      c.ptr(beta, h, "beta") && c.ptr(u, ne, "u") && c.ptr(z, ne, "z") && c.ptr(mean, n, "mean") &&
      c.ptr(rstd, n, "rstd");
  if (c.status) return c.status;
  hipError_t e = tp_launch_sp_ln_fwd(n, h, 1.f / (1.f - p), eps, y, x, mask, gamma, beta, u, z, mean, rstd,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_sp_ln_fwd: %s", hipGetErrorString(e));
  return ok();
}

size_t tp_sp_ln_bwd_workspace(int dt, int64_t n, int64_t h) {
  Checker c;
  c.dtype(dt, false, "tp_sp_ln_bwd_workspace");
  c.dim(n, "n") && c.dim(h, "h");
  if (c.status) return 0;
  return align256((size_t)tp_sp_ln_bwd_grid(n, h) * 2 * h * sizeof(float));
}

int tp_sp_ln_bwd(int dt, int64_t n, int64_t h, float p, const void *dz, const void *dun, const void *u,
                 const float *mean, const float *rstd, const void *gamma, const uint8_t *mask, void *dx, void *dy,
                 void *dgamma, void *dbeta, void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  int64_t ne;
  c.dtype(dt, false, "tp_sp_ln_bwd");
  c.dim(n, "n") && c.dim(h, "h");
  if (!c.status && !(p >= 0.f && p < 1.f)) c.status = fail(TP_EINVAL, "tp_sp_ln_bwd: dropout p = %g not in [0, 1)", p);
  if (!c.status && tp_sp_ln_passes(h) > 2) c.status = fail(TP_EUNSUPPORTED, "tp_sp_ln_bwd: h = %lld > 16384", (long long)h);
  c.elems(n, h, ne, "dz");
  c.ptr(dz, ne, "dz") && c.ptr(dun, ne, "dun") && c.ptr(u, ne, "u") && c.ptr(mean, n, "mean") &&
      c.ptr(rstd, n, "rstd") && c.ptr(gamma, h, "gamma") && c.ptr(mask, ne, "mask") && c.ptr(dx, ne, "dx") &&
      c.ptr(dy, ne, "dy") && c.ptr(dgamma, h, "dgamma") && c.ptr(dbeta, h, "dbeta");
  if (c.status) return c.status;
  ws_ok(c, ws, ws_bytes, h ? align256((size_t)tp_sp_ln_bwd_grid(n, h) * 2 * h * sizeof(float)) : 0, "tp_sp_ln_bwd");
  if (c.status) return c.status;
  hipError_t e = tp_launch_sp_ln_bwd(n, h, 1.f / (1.f - p), dz, dun, u, mean, rstd, gamma, mask, dx, dy, dgamma,
                                     dbeta, (float *)ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_sp_ln_bwd: %s", hipGetErrorString(e));
  return ok();
}

size_t tp_lm_head_ce_workspace(int dt, int64_t s, int64_t h, int64_t Vs) {
  Checker c;
  c.dtype(dt, false, "tp_lm_head_ce_workspace");
  c.dim(s, "s") && c.dim(h, "h") && c.dim(Vs, "Vs");
  if (c.status) return 0;
  return lm_ce_plan(s, h, Vs).bytes;
}

}  // extern "C"

namespace {

// Argument checks shared by the fused LM head + CE calls.
int lm_ce_check(Checker &c, const char *call, int dt, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start,
                const void *Hf, const void *Wlm, const int64_t *target, float *lmax, float *lsumexp, float *tlogit) {
  int64_t nh, nw;
  c.dtype(dt, false, call);
  c.dim(s, "s") && c.dim(h, "h") && c.dim(Vs, "Vs");
  if (!c.status && vocab_start < 0) c.status = fail(TP_ESHAPE, "vocab_start = %lld < 0", (long long)vocab_start);
  c.elems(s, h, nh, "Hf") && c.elems(h, Vs, nw, "Wlm");
  c.ptr(Hf, nh, "Hf") && c.ptr(Wlm, nw, "Wlm") && c.ptr(target, s, "target") && c.ptr(lmax, s, "lmax") &&
      c.ptr(lsumexp, s, "lsumexp") && c.ptr(tlogit, s, "tlogit");
  return c.status;
}

// The GEMM with the CE-statistics epilogue, then the merge of the parts; ws
// holds the plan's partial statistics (every slot the merge reads is written
// by the GEMM of the same call, so ws needs no clearing).
int lm_ce_launch(const LmCePlan &L, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start, const void *Hf,
                 const void *Wlm, const int64_t *target, float *lmax, float *lsumexp, float *tlogit, void *ws,
                 hipStream_t st, const char *call) {
  Ptrs q;
  q.A[0] = Hf; q.lda[0] = h;
  q.B[0] = Wlm; q.ldb[0] = Vs;
  q.ai0 = target;
  GemmDesc d = make_desc(L.g, q, L.p, TP_DT_BF16, ws);
  d.vstart = vocab_start;
  hipError_t e = tp_launch_gemm_bf16(d, variant(L.g, L.p), st);
  if (e == hipSuccess)
    e = tp_launch_ce_merge((const float *)ws, L.parts, s, Vs, vocab_start, target, lmax, lsumexp, tlogit, st);
  if (e != hipSuccess) return fail(TP_EHIP, "%s: %s", call, hipGetErrorString(e));
  return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch`, or an error status
int scratch_ptr(void **out, const char *call) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TP_EHIP, "%s: hipGetDevice: %s", call, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_EUNSUPPORTED, "%s: device %d beyond %d", call, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TP_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", call, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_lm_head_ce_fwd(int dt, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start, const void *Hf,
                      const void *Wlm, const int64_t *target, float *lmax, float *lsumexp, float *tlogit,
                      void *ws, size_t ws_bytes, void *stream) {
  Checker c;
  if (lm_ce_check(c, "tp_lm_head_ce_fwd", dt, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp, tlogit))
    return c.status;
  const LmCePlan L = lm_ce_plan(s, h, Vs);
  ws_ok(c, ws, ws_bytes, L.bytes, "tp_lm_head_ce_fwd");
  if (c.status) return c.status;
  return lm_ce_launch(L, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp, tlogit, ws, (hipStream_t)stream,
                      "tp_lm_head_ce_fwd");
}

size_t tp_lm_head_ce_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int tp_lm_head_ce_fwd_noalloc(int dt, int64_t s, int64_t h, int64_t Vs, int64_t vocab_start, const void *Hf,
                              const void *Wlm, const int64_t *target, float *lmax, float *lsumexp, float *tlogit,
                              void *stream) {
  Checker c;
  if (lm_ce_check(c, "tp_lm_head_ce_fwd_noalloc", dt, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp,
                  tlogit))
    return c.status;
  const LmCePlan L = lm_ce_plan(s, h, Vs);
  if (L.bytes > kNoAllocScratchBytes)
    return fail(TP_EWORKSPACE, "tp_lm_head_ce_fwd_noalloc: s = %lld, Vs = %lld need %zu bytes of scratch; the "
                "allocation-free call holds %zu (use tp_lm_head_ce_fwd with a workspace)", (long long)s,
                (long long)Vs, L.bytes, kNoAllocScratchBytes);
  if (s == 0) return ok();
  void *ws = nullptr;
  if (int e = scratch_ptr(&ws, "tp_lm_head_ce_fwd_noalloc")) return e;
  return lm_ce_launch(L, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp, tlogit, ws, (hipStream_t)stream,
                      "tp_lm_head_ce_fwd_noalloc");
}

int tp_vocab_embed(int dt, int64_t n, int64_t Vs, int64_t h, int64_t vocab_start, const int64_t *ids,
                   const void *table, void *out, void *stream) {
  Checker c;
  int64_t nt, no;
  c.dtype(dt, true, "tp_vocab_embed");
  c.dim(n, "n") && c.dim(Vs, "Vs") && c.dim(h, "h");
  if (!c.status && vocab_start < 0) c.status = fail(TP_ESHAPE, "vocab_start = %lld < 0", (long long)vocab_start);
  c.elems(Vs, h, nt, "table") && c.elems(n, h, no, "out");
  c.ptr(ids, n, "ids") && c.ptr(table, nt, "table") && c.ptr(out, no, "out");
  if (c.status) return c.status;
  hipError_t e = tp_launch_vocab_embed((int)esize(dt), n, Vs, h, vocab_start, ids, table, out,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_EHIP, "tp_vocab_embed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
