// spec_verify.hip -- speculative-sampling verification for gfx950 (MI355X).
//
// One persistent, cooperatively launched kernel runs the whole step.  The
// vocabulary of every row is cut into fixed tiles of TILE elements.  A work
// item is one tile of one "group": for i < k the group is the pair (target row
// i, draft row i) of a sequence, and group k is the target row k alone (in
// greedy mode every group is a single target row).  Workgroups take items
// round-robin (item = blockIdx.x + r * gridDim.x); the items of a group are
// consecutive, so a group is always spread over distinct, co-resident
// workgroups.
//
// Per item:
//  A  stream the tile(s) into registers with 128-bit loads, compute per-thread
//     max and sum of exp2((x - max) * log2(e)/T) (fp32 exp, per-thread fp32
//     sums, fp64 above that), reduce to a tile record; publish it.
//  -- group barrier: wait until every tile of the group has published.
//  B  combine the tile records in tile order (fp64) into the row max and
//     normaliser, identical in every workgroup of the group; compute the tile's
//     residual mass sum max(0, p - q) (or p for row k) from the resident tile and
//     publish it; filter the tile's top-32 candidates against a row bound (the
//     32nd largest wave maximum: at least 32 elements lie at or above it) and
//     append them; tile 0 also takes the acceptance decision of the row.
//  C  the last workgroup of the group to finish merges the candidates into the
//     top-32 (value desc, index asc) and, if it is also the last group of the
//     sequence, assembles the sequence: first rejection j, then an inverse-CDF
//     draw over the tile masses of row j in tile order, the crossing tile
//     re-read and scanned element by element.
//
// Acceptance test, residual and bonus draw follow the ReSpec notes ("2 .
// background": one-shot acceptance test Eq.1, residual max(0,p-q)/sum); the
// procedure order follows the ReSpec blog (speculative-decoding steps 1-4); the
// top-32 soft targets follow the ReSpec notes ("4 . G2" worked example).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "spec_verify.h"

namespace {

constexpr int TPB = 256;               // threads per workgroup (4 waves of 64)
constexpr int NWAVE = TPB / 64;
constexpr int EPT = 16;                // elements per thread per row
constexpr int TILE = TPB * EPT;        // 4096 vocabulary entries per tile
constexpr int CAP = 512;               // candidate slots per target row
constexpr int TOPK = SV_TOPK;
constexpr int MAX_TILES = 256;         // V <= MAX_TILES * TILE
constexpr uint32_t SPIN_LIMIT = 1u << 19;      // about half a second of polling
constexpr float NEG_INF = -__builtin_inff();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Fmt;
template <> struct Fmt<SV_BF16> { static constexpr int E = 2, W = 8, NSEG = 2; };
template <> struct Fmt<SV_F32> { static constexpr int E = 4, W = 4, NSEG = 4; };

// Published per (group, tile) after phase A.
struct TileRec {
  float m_t, m_d;          // tile max of the target / draft row part
  double s_t, s_d;         // sum exp2((x - m) * sc) over the tile part
  uint32_t wkey[NWAVE];    // ordered key of each wave's target maximum, 0 = no element
  int32_t flags_t, flags_d;
};

// Published per group by its tile-0 workgroup in phase B.
struct GroupRec {
  double s_t, s_d;         // row normalisers (relative to m_t, m_d)
  float m_t, m_d;          // row maxima
  int32_t flags;           // SV_STATUS_* bits of this group's rows and token
  int32_t accept;          // 1 when the drafted token passed (pair groups)
  int32_t nan_t;           // the target row holds a NaN
  int32_t pad;
};

struct GroupSync { int32_t arrive1, arrive2, ncand, pad; };

struct Params {
  const char *target, *draft;
  int64_t tstride, dstride;            // row strides in elements
  const int32_t *tokens;
  const float *uniforms;
  int32_t *accepted_len, *out_tokens, *topk_idx, *status;
  float *topk_val, *lse_t, *lse_d, *p_tok, *q_tok;
  GroupSync *sync;
  int32_t *seqctr, *fault;
  TileRec *recs;
  double *rsum;
  GroupRec *grec;
  uint64_t *cand;
  int32_t B, k, V, nT, items;
  int32_t cap;                         // candidate slots per target row: min(CAP, V)
  float T, sc;                         // sc = log2(e) / T
  double scd;
  int32_t t_vec, d_vec;                // rows 16-byte aligned
};

struct Smem {
  float f[4][NWAVE];
  uint32_t u[2][NWAVE];
  int32_t i[4][NWAVE];
  double d[4][NWAVE];
  int32_t bc[8];
  double dbc[4];
  union {
    uint32_t wkeys[4 * MAX_TILES];     // phase B: wave maxima of the row
    uint64_t keys[CAP];                // group finalise: candidate keys
    struct {                           // exact top-32 fallback
      uint32_t hist[2048];
      int32_t part[TPB];
      uint64_t list[TOPK];
    } fb;
    double tot[MAX_TILES];             // residual fallback: per-tile masses
  };
};

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;                       // -0.0 ties +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// larger = earlier in (value desc, index asc)
__device__ __forceinline__ uint64_t cand_key(float v, int32_t x) {
  return ((uint64_t)ordered_key(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)x);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { uint32_t w = __shfl_xor(v, o); v = w > v ? w : v; }
  return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_incl_int(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) { int w = __shfl_up(v, d); if (lane >= d) v += w; }
  return v;
}
__device__ __forceinline__ double wave_incl_dbl(double v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) { double w = __shfl_up(v, d); if (lane >= d) v += w; }
  return v;
}

__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ int ld_relaxed(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_acq_rel(int32_t *p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT> __device__ __forceinline__ float load_elem(const char *row, int64_t x) {
  if constexpr (DT == SV_BF16) {
    return __uint_as_float((uint32_t)(*(const uint16_t *)(row + x * 2)) << 16);
  } else {
    return *(const float *)(row + x * 4);
  }
}

template <int DT> __device__ __forceinline__ float elem(const u32x4 (&r)[Fmt<DT>::NSEG], int s, int w) {
  if constexpr (DT == SV_BF16) {
    uint32_t word = r[s][w >> 1];
    return __uint_as_float((w & 1) ? (word & 0xffff0000u) : (word << 16));
  } else {
    return __uint_as_float(r[s][w]);
  }
}

// tile-local position of element (s, w) of this thread
template <int DT> __device__ __forceinline__ int tpos(int s, int w) {
  return s * (TPB * Fmt<DT>::W) + (int)threadIdx.x * Fmt<DT>::W + w;
}

// Stream one tile of a row into registers; entries past V read as -inf.
template <int DT>
__device__ __forceinline__ void load_tile(const char *row, int c, int V, bool vec, u32x4 (&r)[Fmt<DT>::NSEG]) {
  constexpr int E = Fmt<DT>::E, W = Fmt<DT>::W, NSEG = Fmt<DT>::NSEG;
  const int64_t c0 = (int64_t)c * TILE;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const int64_t e0 = c0 + s * (TPB * W) + (int64_t)threadIdx.x * W;
    if (vec && e0 + W <= V) {
      r[s] = __builtin_nontemporal_load((const u32x4 *)(row + e0 * E));
    } else {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (DT == SV_BF16) {
          const int64_t x = e0 + 2 * q;
          uint32_t lo = x < V ? *(const uint16_t *)(row + x * 2) : 0xff80u;
          uint32_t hi = x + 1 < V ? *(const uint16_t *)(row + (x + 1) * 2) : 0xff80u;
          v[q] = lo | (hi << 16);
        } else {
          const int64_t x = e0 + q;
          v[q] = x < V ? *(const uint32_t *)(row + x * 4) : 0xff800000u;
        }
      }
      r[s] = v;
    }
  }
}

// Per-thread max, and with EXPS the terms e = exp2((x - m) * sc) and their
// sequential fp32 sum.  flags gets SV_STATUS_NAN / SV_STATUS_POSINF.
template <int DT, bool EXPS>
__device__ __forceinline__ void thread_stats(const u32x4 (&r)[Fmt<DT>::NSEG], float sc, float (&e)[EPT],
                                             float &m, float &s, int &flags) {
  constexpr int W = Fmt<DT>::W, NSEG = Fmt<DT>::NSEG;
  m = NEG_INF;
#pragma unroll
  for (int g = 0; g < NSEG; ++g)
#pragma unroll
    for (int w = 0; w < W; ++w) m = fmaxf(m, elem<DT>(r, g, w));
  flags = 0;
  s = 0.f;
  if constexpr (EXPS) {
    const float ms = (m == NEG_INF) ? 0.f : m;
#pragma unroll
    for (int g = 0; g < NSEG; ++g)
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float t = __builtin_amdgcn_exp2f((elem<DT>(r, g, w) - ms) * sc);
        e[g * W + w] = t;
        s += t;
      }
    if (!(s == s)) {            // NaN or +inf somewhere in this thread's slice
      bool nan = false;
#pragma unroll
      for (int g = 0; g < NSEG; ++g)
#pragma unroll
        for (int w = 0; w < W; ++w) { float x = elem<DT>(r, g, w); nan |= !(x == x); }
      flags = nan ? SV_STATUS_NAN : SV_STATUS_POSINF;
    }
  } else {
    bool nan = false;
#pragma unroll
    for (int g = 0; g < NSEG; ++g)
#pragma unroll
      for (int w = 0; w < W; ++w) { float x = elem<DT>(r, g, w); nan |= !(x == x); }
    flags = nan ? SV_STATUS_NAN : 0;
  }
}

// Per-thread scale turning e into probabilities: exp2((m_thread - m_row) * sc) / s_row.
__device__ __forceinline__ float prob_scale(float m_thr, float m_row, double s_row, float sc) {
  if (m_thr == NEG_INF) return 0.f;
  return (float)((double)__builtin_amdgcn_exp2f((m_thr - m_row) * sc) / s_row);
}

// Mass of one element: residual max(0, p - q) for pair rows, p otherwise.
__device__ __forceinline__ float mass_of(float et, float at, float ed, float ad, bool resid) {
  const float p = et * at;
  if (!resid) return p;
  const float q = ed * ad;
  const float r = p - q;
  return r > 0.f ? r : 0.f;
}

// Exclusive prefix (fp64) of per-thread segment masses over the tile, in the
// tile's element order (segment-major, then thread).  base[s] receives the
// mass of all tile elements before this thread's segment s; returns the tile
// total.  Fixed association: identical bits wherever it is evaluated.
template <int NSEG>
__device__ double tile_scan(const float (&seg)[NSEG], double (&base)[NSEG], Smem &sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  double acc = 0.0;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const double x = (double)seg[s];
    const double inc = wave_incl_dbl(x, lane);
    double prev = __shfl_up(inc, 1);
    if (lane == 0) prev = 0.0;
    if (lane == 63) sm.d[s & 3][wid] = inc;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wid; ++w) off += sm.d[s & 3][w];
    double tot = 0.0;
    for (int w = 0; w < NWAVE; ++w) tot += sm.d[s & 3][w];
    base[s] = acc + (off + prev);
    acc = acc + tot;
    if ((s & 3) == 3) __syncthreads();
  }
  __syncthreads();
  return acc;
}

// Top-32 of a target row by exact radix selection over the whole row (used
// when the candidate filter overflowed or the row is too short for the bound).
template <int DT>
__device__ __forceinline__ void topk_exact(const char *row, int V, float *oval, int32_t *oidx, Smem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int need = V < TOPK ? V : TOPK;
  uint32_t prefix = 0, pmask = 0;
  int above = 0;                               // keys strictly above the prefix bucket
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int h = tid; h < 2048; h += TPB) sm.fb.hist[h] = 0;
    __syncthreads();
    for (int x = tid; x < V; x += TPB) {
      const uint32_t key = ordered_key(load_elem<DT>(row, x));
      if ((key & pmask) == prefix) atomicAdd(&sm.fb.hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // per-thread totals of nb/TPB consecutive bins, then the bucket holding the
    // (need - above)-th largest key among those matching the prefix
    const int per = nb / TPB;
    int local = 0;
    for (int h = 0; h < per; ++h) local += (int)sm.fb.hist[tid * per + h];
    sm.fb.part[tid] = local;
    __syncthreads();
    if (tid == 0) {
      const int want = need - above;
      int cum = 0, t = TPB - 1;
      for (; t > 0; --t) {
        if (cum + sm.fb.part[t] >= want) break;
        cum += sm.fb.part[t];
      }
      int h = t * per + per - 1;
      for (; h > t * per; --h) {
        if (cum + (int)sm.fb.hist[h] >= want) break;
        cum += (int)sm.fb.hist[h];
      }
      sm.bc[0] = h;
      sm.bc[1] = above + cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.bc[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    above = sm.bc[1];
    __syncthreads();
  }
  // prefix is now the key of the need-th largest element; `above` keys exceed it
  const uint32_t theta = prefix;
  const int eq_need = need - above;
  if (tid == 0) { sm.bc[2] = 0; sm.bc[3] = 0; }
  __syncthreads();
  for (int x0 = 0; x0 < V; x0 += TPB) {
    const int x = x0 + tid;
    uint32_t key = 0;
    if (x < V) key = ordered_key(load_elem<DT>(row, x));
    if (x < V && key > theta) {
      const int slot = atomicAdd(&sm.bc[2], 1);
      sm.fb.list[slot] = ((uint64_t)key << 32) | (0xffffffffu - (uint32_t)x);
    }
    const bool eq = x < V && key == theta;
    const uint64_t bal = __ballot(eq);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sm.i[0][wid] = __popcll(bal);
    __syncthreads();
    int woff = sm.bc[3];
    for (int w = 0; w < wid; ++w) woff += sm.i[0][w];
    const int rank = woff + before;
    if (eq && rank < eq_need) sm.fb.list[above + rank] = ((uint64_t)key << 32) | (0xffffffffu - (uint32_t)x);
    __syncthreads();
    if (tid == 0) for (int w = 0; w < NWAVE; ++w) sm.bc[3] += sm.i[0][w];
    __syncthreads();
    if (sm.bc[3] >= eq_need && sm.bc[2] == above) break;
  }
  __syncthreads();
  // `need` unique keys: rank by counting, write in order
  if (tid < need) {
    const uint64_t ka = sm.fb.list[tid];
    int rank = 0;
    for (int j = 0; j < need; ++j) rank += sm.fb.list[j] > ka;
    const int32_t x = (int32_t)(0xffffffffu - (uint32_t)ka);
    oidx[rank] = x;
    oval[rank] = load_elem<DT>(row, x);
  }
  for (int r = need + tid; r < TOPK; r += TPB) { oidx[r] = -1; oval[r] = NEG_INF; }
  __syncthreads();
}

// Draw by inverse CDF inside one tile: the first element (ascending index) of
// positive mass whose cumulative mass prefix + (scan base + running fp32 sum)
// exceeds tau; if rounding leaves none, the tile's last positive-mass element.
template <int DT>
__device__ int tile_draw(const char *trow, const char *drow, int c, const Params &P, bool resid,
                         float m_t, double s_t, float m_d, double s_d, double prefix, double tau, Smem &sm) {
  constexpr int W = Fmt<DT>::W, NSEG = Fmt<DT>::NSEG;
  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(trow, c, P.V, P.t_vec, rt);
  if (resid) load_tile<DT>(drow, c, P.V, P.d_vec, rd);
  float et[EPT], ed[EPT], mt, st, md = NEG_INF, sd;
  int ft, fd;
  thread_stats<DT, true>(rt, P.sc, et, mt, st, ft);
  if (resid) thread_stats<DT, true>(rd, P.sc, ed, md, sd, fd);
  const float at = prob_scale(mt, m_t, s_t, P.sc);
  const float ad = resid ? prob_scale(md, m_d, s_d, P.sc) : 0.f;
  float seg[NSEG];
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) a += mass_of(et[g * W + w], at, resid ? ed[g * W + w] : 0.f, ad, resid);
    seg[g] = a;
  }
  double base[NSEG];
  tile_scan<NSEG>(seg, base, sm);
  int first = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mval = mass_of(et[g * W + w], at, resid ? ed[g * W + w] : 0.f, ad, resid);
      a += mval;
      const int pos = tpos<DT>(g, w);
      if (mval > 0.f) {
        lastpos = pos > lastpos ? pos : lastpos;
        if (prefix + (base[g] + (double)a) > tau && pos < first) first = pos;
      }
    }
  }
  // block min of `first`, block max of `lastpos`
  for (int o = 32; o > 0; o >>= 1) {
    int f2 = __shfl_xor(first, o), l2 = __shfl_xor(lastpos, o);
    first = f2 < first ? f2 : first;
    lastpos = l2 > lastpos ? l2 : lastpos;
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sm.i[2][wid] = first; sm.i[3][wid] = lastpos; }
  __syncthreads();
  int f = sm.i[2][0], l = sm.i[3][0];
  for (int w = 1; w < NWAVE; ++w) {
    f = sm.i[2][w] < f ? sm.i[2][w] : f;
    l = sm.i[3][w] > l ? sm.i[3][w] : l;
  }
  __syncthreads();
  const int pos = f != 0x7fffffff ? f : l;
  return pos < 0 ? -1 : c * TILE + pos;
}

// Total mass of one tile (same arithmetic as tile_draw).
template <int DT>
__device__ double tile_mass(const char *trow, const char *drow, int c, const Params &P, bool resid,
                            float m_t, double s_t, float m_d, double s_d, Smem &sm) {
  constexpr int W = Fmt<DT>::W, NSEG = Fmt<DT>::NSEG;
  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(trow, c, P.V, P.t_vec, rt);
  if (resid) load_tile<DT>(drow, c, P.V, P.d_vec, rd);
  float et[EPT], ed[EPT], mt, st, md = NEG_INF, sd;
  int ft, fd;
  thread_stats<DT, true>(rt, P.sc, et, mt, st, ft);
  if (resid) thread_stats<DT, true>(rd, P.sc, ed, md, sd, fd);
  const float at = prob_scale(mt, m_t, s_t, P.sc);
  const float ad = resid ? prob_scale(md, m_d, s_d, P.sc) : 0.f;
  float seg[NSEG];
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) a += mass_of(et[g * W + w], at, resid ? ed[g * W + w] : 0.f, ad, resid);
    seg[g] = a;
  }
  double base[NSEG];
  return tile_scan<NSEG>(seg, base, sm);
}

// Sampling-mode sequence assembly (run by the last group of the sequence).
template <int DT>
__device__ __forceinline__ void finish_sampling(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1, nT = P.nT;
  if (tid == 0) {
    int st = 0, j = k;
    for (int i = 0; i <= k; ++i) {
      const GroupRec &r = P.grec[b * K1 + i];
      st |= r.flags;
      if (i < k && j == k && !r.accept) j = i;
    }
    for (int i = 0; i < k + 2; ++i) {
      const float u = P.uniforms[(int64_t)b * (k + 2) + i];
      if (!(u >= 0.f && u < 1.f)) st |= SV_STATUS_BAD_UNIFORM;
    }
    if (ld_relaxed(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
    int cstar = -1;
    double prefix = 0.0, tau = 0.0;
    if (!st) {
      const int g = b * K1 + j;
      const double u = (double)P.uniforms[(int64_t)b * (k + 2) + (j < k ? k : k + 1)];
      double R = 0.0;
      for (int c = 0; c < nT; ++c) R += P.rsum[(int64_t)g * nT + c];
      tau = u * R;
      double Pc = 0.0;
      for (int c = 0; c < nT; ++c) {
        const double nx = Pc + P.rsum[(int64_t)g * nT + c];
        if (nx > tau) { cstar = c; break; }
        Pc = nx;
      }
      prefix = Pc;
    }
    sm.bc[0] = st;
    sm.bc[1] = j;
    sm.bc[2] = cstar;
    sm.dbc[0] = prefix;
    sm.dbc[1] = tau;
  }
  __syncthreads();
  const int st = sm.bc[0], j = sm.bc[1];
  int cstar = sm.bc[2];
  double prefix = sm.dbc[0], tau = sm.dbc[1];
  __syncthreads();
  int token = -1;
  if (!st) {
    const int g = b * K1 + j;
    const bool resid = j < k;
    const GroupRec gr = P.grec[g];
    const char *trow = P.target + ((int64_t)b * K1 + j) * P.tstride * Fmt<DT>::E;
    const char *drow = resid ? P.draft + ((int64_t)b * k + j) * P.dstride * Fmt<DT>::E : nullptr;
    bool use_p = false;
    if (cstar < 0) {
      // no residual mass left (rounding): draw from p_j with the same uniform
      use_p = true;
      for (int c = 0; c < nT; ++c) {
        const double m = tile_mass<DT>(trow, nullptr, c, P, false, gr.m_t, gr.s_t, 0.f, 1.0, sm);
        if (tid == 0) sm.tot[c] = m;
      }
      __syncthreads();
      if (tid == 0) {
        const double u = (double)P.uniforms[(int64_t)b * (k + 2) + (j < k ? k : k + 1)];
        double R = 0.0;
        for (int c = 0; c < nT; ++c) R += sm.tot[c];
        const double tu = u * R;
        double Pc = 0.0;
        int cs = nT - 1;
        for (int c = 0; c < nT; ++c) {
          const double nx = Pc + sm.tot[c];
          if (nx > tu) { cs = c; break; }
          Pc = nx;
        }
        sm.bc[2] = cs;
        sm.dbc[0] = Pc;
        sm.dbc[1] = tu;
      }
      __syncthreads();
      cstar = sm.bc[2];
      prefix = sm.dbc[0];
      tau = sm.dbc[1];
      __syncthreads();
    }
    token = tile_draw<DT>(trow, drow, cstar, P, resid && !use_p, gr.m_t, gr.s_t, gr.m_d, gr.s_d, prefix, tau, sm);
  }
  if (tid == 0) {
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
  }
  for (int i = tid; i < K1; i += TPB) {
    int v = -1;
    if (!st) v = i < j ? P.tokens[(int64_t)b * k + i] : (i == j ? token : -1);
    P.out_tokens[(int64_t)b * K1 + i] = v;
  }
}

// Greedy-mode sequence assembly: argmax-prefix match on the top-1 entries.
__device__ __forceinline__ void finish_greedy(const Params &P, int b) {
  const int k = P.k, K1 = k + 1;
  if (threadIdx.x == 0) {
    int st = 0, j = k;
    for (int i = 0; i <= k; ++i) st |= P.grec[b * K1 + i].flags;
    for (int i = 0; i < k; ++i) {
      const int32_t x = P.tokens[(int64_t)b * k + i];
      if (x < 0 || x >= P.V) st |= SV_STATUS_BAD_TOKEN;
    }
    if (ld_relaxed(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
    if (!st)
      for (int i = 0; i < k; ++i)
        if (P.tokens[(int64_t)b * k + i] != P.topk_idx[((int64_t)b * K1 + i) * TOPK]) { j = i; break; }
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
    for (int i = 0; i < K1; ++i) {
      int v = -1;
      if (!st) v = i < j ? P.tokens[(int64_t)b * k + i] : (i == j ? P.topk_idx[((int64_t)b * K1 + j) * TOPK] : -1);
      P.out_tokens[(int64_t)b * K1 + i] = v;
    }
  }
}

template <int DT, bool GREEDY>
__device__ __forceinline__ void process_item(const Params &P, int item, Smem &sm) {
  constexpr int E = Fmt<DT>::E, W = Fmt<DT>::W, NSEG = Fmt<DT>::NSEG;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1, V = P.V;
  const int g = item / nT, c = item - g * nT;
  const int b = g / K1, i = g - b * K1;
  const bool pair = !GREEDY && i < k;
  const char *trow = P.target + ((int64_t)b * K1 + i) * P.tstride * E;
  const char *drow = pair ? P.draft + ((int64_t)b * k + i) * P.dstride * E : nullptr;

  // drafted token and its two logits, for the row's acceptance decision
  int32_t x = -1;
  float tx = 0.f, dx = 0.f;
  if (pair && c == 0 && tid == 0) {
    x = P.tokens[(int64_t)b * k + i];
    if (x >= 0 && x < V) { tx = load_elem<DT>(trow, x); dx = load_elem<DT>(drow, x); }
  }

  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(trow, c, V, P.t_vec, rt);
  if (pair) load_tile<DT>(drow, c, V, P.d_vec, rd);

  // ---------------- phase A: per-thread and per-tile statistics
  float et[EPT], ed[EPT];
  float mt, st, md = NEG_INF, sd = 0.f;
  int ft, fd = 0;
  thread_stats<DT, !GREEDY>(rt, P.sc, et, mt, st, ft);
  if (pair) thread_stats<DT, true>(rd, P.sc, ed, md, sd, fd);
  const bool has_elem = (int64_t)c * TILE + (int64_t)tid * W < V;
  const uint32_t tkey = has_elem ? ordered_key(mt) : 0u;

  {
    const float wm_t = wave_max(mt), wm_d = wave_max(md);
    const uint32_t wk = wave_max_u(tkey);
    const int wf_t = wave_or(ft), wf_d = wave_or(fd);
    if (lane == 0) { sm.f[0][wid] = wm_t; sm.f[1][wid] = wm_d; sm.u[0][wid] = wk; sm.i[0][wid] = wf_t; sm.i[1][wid] = wf_d; }
  }
  __syncthreads();
  float m_ct = sm.f[0][0], m_cd = sm.f[1][0];
  int f_ct = sm.i[0][0], f_cd = sm.i[1][0];
  for (int w = 1; w < NWAVE; ++w) {
    m_ct = fmaxf(m_ct, sm.f[0][w]); m_cd = fmaxf(m_cd, sm.f[1][w]);
    f_ct |= sm.i[0][w]; f_cd |= sm.i[1][w];
  }
  double s_ct = 0.0, s_cd = 0.0;
  if (!GREEDY) {
    double a = (mt == NEG_INF) ? 0.0 : (double)st * (double)__builtin_amdgcn_exp2f((mt - m_ct) * P.sc);
    double d = 0.0;
    if (pair) d = (md == NEG_INF) ? 0.0 : (double)sd * (double)__builtin_amdgcn_exp2f((md - m_cd) * P.sc);
    a = wave_sum(a);
    d = wave_sum(d);
    if (lane == 0) { sm.d[0][wid] = a; sm.d[1][wid] = d; }
    __syncthreads();
    for (int w = 0; w < NWAVE; ++w) { s_ct += sm.d[0][w]; s_cd += sm.d[1][w]; }
  }
  if (tid == 0) {
    TileRec r;
    r.m_t = m_ct; r.m_d = m_cd; r.s_t = s_ct; r.s_d = s_cd;
    for (int w = 0; w < NWAVE; ++w) r.wkey[w] = sm.u[0][w];
    r.flags_t = f_ct; r.flags_d = f_cd;
    P.recs[item] = r;
  }

  // ---------------- group barrier: every tile of the group has published
  __syncthreads();
  if (tid == 0) {
    GroupSync *gs = P.sync + g;
    fence_release();
    const int old1 = add_acq_rel(&gs->arrive1, 1);
    if (old1 < 0 || old1 >= nT) atomicOr(P.fault, 2);
    uint32_t spins = 0;
    while (ld_relaxed(&gs->arrive1) < nT) {
      __builtin_amdgcn_s_sleep(2);
      // a wait that never ends would be a bug: give up, mark the fault, and let
      // every later wait give up at once so the grid drains
      if (++spins > SPIN_LIMIT || ((spins & 255) == 0 && ld_relaxed(P.fault))) {
        atomicOr(P.fault, 1);
        break;
      }
    }
  }
  __syncthreads();
  fence_acquire();

  // ---------------- phase B: row statistics, identical in every workgroup
  float m_rt = NEG_INF, m_rd = NEG_INF;
  int f_rt = 0, f_rd = 0;
  for (int cc = tid; cc < nT; cc += TPB) {
    const TileRec &r = P.recs[(int64_t)g * nT + cc];
    m_rt = fmaxf(m_rt, r.m_t); m_rd = fmaxf(m_rd, r.m_d);
    f_rt |= r.flags_t; f_rd |= r.flags_d;
    for (int w = 0; w < NWAVE; ++w) sm.wkeys[cc * NWAVE + w] = r.wkey[w];
  }
  {
    const float a = wave_max(m_rt), d = wave_max(m_rd);
    const int fa = wave_or(f_rt), fb = wave_or(f_rd);
    if (lane == 0) { sm.f[2][wid] = a; sm.f[3][wid] = d; sm.i[2][wid] = fa; sm.i[3][wid] = fb; }
  }
  __syncthreads();
  m_rt = sm.f[2][0]; m_rd = sm.f[3][0]; f_rt = sm.i[2][0]; f_rd = sm.i[3][0];
  for (int w = 1; w < NWAVE; ++w) {
    m_rt = fmaxf(m_rt, sm.f[2][w]); m_rd = fmaxf(m_rd, sm.f[3][w]);
    f_rt |= sm.i[2][w]; f_rd |= sm.i[3][w];
  }
  double s_rt = 0.0, s_rd = 0.0;
  if (!GREEDY) {
    double a = 0.0, d = 0.0;
    for (int cc = tid; cc < nT; cc += TPB) {
      const TileRec &r = P.recs[(int64_t)g * nT + cc];
      if (r.m_t != NEG_INF) a += r.s_t * (double)__builtin_amdgcn_exp2f((r.m_t - m_rt) * P.sc);
      if (pair && r.m_d != NEG_INF) d += r.s_d * (double)__builtin_amdgcn_exp2f((r.m_d - m_rd) * P.sc);
    }
    a = wave_sum(a);
    d = wave_sum(d);
    if (lane == 0) { sm.d[2][wid] = a; sm.d[3][wid] = d; }
  }
  // row bound for top-32 candidates: the 32nd largest wave maximum (0 when
  // fewer than 32 waves hold elements: every element is then a candidate)
  if (wid == 0) {
    const int nkeys = nT * NWAVE;
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int cnt = 0;
      for (int j0 = 0; j0 < nkeys; j0 += 64) {
        const int j = j0 + lane;
        cnt += __popcll(__ballot(j < nkeys && sm.wkeys[j] >= cand));
      }
      if (cnt >= TOPK) prefix = cand;
    }
    if (lane == 0) sm.u[1][0] = prefix;
  }
  __syncthreads();
  if (!GREEDY) for (int w = 0; w < NWAVE; ++w) { s_rt += sm.d[2][w]; s_rd += sm.d[3][w]; }
  const uint32_t L = sm.u[1][0];
  // one data-error bit per row: NaN before +inf before an empty row
  f_rt = (f_rt & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rt;
  f_rd = (f_rd & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rd;
  if (m_rt == NEG_INF && !f_rt && !GREEDY) f_rt = SV_STATUS_EMPTY_ROW;
  if (pair && m_rd == NEG_INF && !f_rd) f_rd = SV_STATUS_EMPTY_ROW;

  // acceptance decision of the row (tile 0, one thread)
  if (c == 0 && tid == 0) {
    GroupRec gr;
    gr.s_t = s_rt; gr.s_d = s_rd; gr.m_t = m_rt; gr.m_d = m_rd;
    gr.nan_t = (f_rt & SV_STATUS_NAN) ? 1 : 0;
    gr.pad = 0;
    int fl = f_rt | (pair ? f_rd : 0);
    if (GREEDY) fl &= SV_STATUS_NAN;
    int acc = 1;
    if (pair) {
      float pt = __builtin_nanf(""), qt = __builtin_nanf("");
      if (x < 0 || x >= V) {
        fl |= SV_STATUS_BAD_TOKEN;
        acc = 0;
      } else if (!fl) {
        const double p = exp2(((double)tx - (double)m_rt) * P.scd) / s_rt;
        const double q = exp2(((double)dx - (double)m_rd) * P.scd) / s_rd;
        const double ratio = q > 0.0 ? p / q : (p > 0.0 ? __builtin_inf() : 0.0);
        const double a = ratio < 1.0 ? ratio : 1.0;
        const double u = (double)P.uniforms[(int64_t)b * (k + 2) + i];
        acc = (u < a) ? 1 : 0;
        pt = (float)p;
        qt = (float)q;
      } else {
        acc = 0;
      }
      if (P.p_tok) P.p_tok[(int64_t)b * k + i] = pt;
      if (P.q_tok) P.q_tok[(int64_t)b * k + i] = qt;
      if (P.lse_d) P.lse_d[(int64_t)b * k + i] = (float)((double)m_rd / (double)P.T + log(s_rd));
    }
    if (!GREEDY && P.lse_t) P.lse_t[(int64_t)b * K1 + i] = (float)((double)m_rt / (double)P.T + log(s_rt));
    gr.flags = fl;
    gr.accept = acc;
    P.grec[g] = gr;
  }

  // residual (pair) or target (row k) mass of this tile, published for the draw
  if (!GREEDY) {
    const float at = prob_scale(mt, m_rt, s_rt, P.sc);
    const float ad = pair ? prob_scale(md, m_rd, s_rd, P.sc) : 0.f;
    float seg[NSEG];
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) a += mass_of(et[s * W + w], at, pair ? ed[s * W + w] : 0.f, ad, pair);
      seg[s] = a;
    }
    double base[NSEG];
    const double tot = tile_scan<NSEG>(seg, base, sm);
    if (tid == 0) P.rsum[item] = tot;
  }

  // top-32 candidates of the target row: elements at or above the bound
  {
    const float Lf = key_value(L);
    const bool maybe = has_elem && (L == 0u || mt >= Lf);
    if (__ballot(maybe) != 0ull) {
      int cnt = 0;
      if (maybe) {
#pragma unroll
        for (int s = 0; s < NSEG; ++s)
#pragma unroll
          for (int w = 0; w < W; ++w) {
            const float v = elem<DT>(rt, s, w);
            const int64_t xg = (int64_t)c * TILE + tpos<DT>(s, w);
            cnt += (xg < V && (L == 0u || v >= Lf)) ? 1 : 0;
          }
      }
      const int inc = wave_incl_int(cnt, lane);
      int basei = 0;
      if (lane == 63 && inc > 0) basei = atomicAdd(&P.sync[g].ncand, inc);
      basei = __shfl(basei, 63);
      int slot = basei + inc - cnt;
      if (cnt) {
        uint64_t *dst = P.cand + (int64_t)g * P.cap;
#pragma unroll
        for (int s = 0; s < NSEG; ++s)
#pragma unroll
          for (int w = 0; w < W; ++w) {
            const float v = elem<DT>(rt, s, w);
            const int64_t xg = (int64_t)c * TILE + tpos<DT>(s, w);
            if (xg < V && (L == 0u || v >= Lf)) {
              if (slot >= 0 && slot < P.cap) dst[slot] = cand_key(v, (int32_t)xg);
              ++slot;
            }
          }
      }
    }
  }

  // ---------------- group arrival; the last workgroup finishes the group
  fence_release();           // candidates were written by many threads
  __syncthreads();
  if (tid == 0) sm.bc[4] = add_acq_rel(&P.sync[g].arrive2, 1);
  __syncthreads();
  if (sm.bc[4] != nT - 1) return;
  fence_acquire();

  // top-32 of target row (b, i)
  {
    float *oval = P.topk_val + ((int64_t)b * K1 + i) * TOPK;
    int32_t *oidx = P.topk_idx + ((int64_t)b * K1 + i) * TOPK;
    if (tid == 0) sm.bc[6] = ld_relaxed(&P.sync[g].ncand);
    __syncthreads();
    const int n = sm.bc[6];
    if (f_rt & SV_STATUS_NAN) {
      for (int r = tid; r < TOPK; r += TPB) { oval[r] = __builtin_nanf(""); oidx[r] = -1; }
    } else if (n >= 0 && n <= P.cap) {
      const uint64_t *src = P.cand + (int64_t)g * P.cap;
      for (int a = tid; a < n; a += TPB) sm.keys[a] = src[a];
      __syncthreads();
      for (int a = tid; a < n; a += TPB) {
        const uint64_t ka = sm.keys[a];
        int rank = 0;
        for (int jj = 0; jj < n; ++jj) rank += sm.keys[jj] > ka;
        if (rank < TOPK) {
          const int32_t xi = (int32_t)(0xffffffffu - (uint32_t)ka);
          oidx[rank] = xi;
          oval[rank] = load_elem<DT>(trow, xi);
        }
      }
      for (int r = n + tid; r < TOPK; r += TPB) { oval[r] = NEG_INF; oidx[r] = -1; }
      __syncthreads();
    } else {
      topk_exact<DT>(trow, V, oval, oidx, sm);
    }
  }
  // Every workgroup of the group is past both barriers and done reading the
  // group's tile records and candidates: clear them, so that each call leaves
  // the whole workspace zero-filled whatever shape the next call has.
  {
    uint64_t *cz = P.cand + (int64_t)g * P.cap;
    const int n = sm.bc[6];
    const int nc = n < 0 || n > P.cap ? P.cap : n;
    __syncthreads();
    for (int a = tid; a < nc; a += TPB) cz[a] = 0;
    uint32_t *rz = (uint32_t *)(P.recs + (int64_t)g * nT);
    const int nw = nT * (int)(sizeof(TileRec) / 4);
    for (int a = tid; a < nw; a += TPB) rz[a] = 0;
  }
  if (tid == 0) {
    st_relaxed(&P.sync[g].arrive1, 0);
    st_relaxed(&P.sync[g].arrive2, 0);
    st_relaxed(&P.sync[g].ncand, 0);
  }

  // ---------------- sequence arrival; the last group assembles the sequence
  fence_release();           // top-32 outputs were written by many threads
  __syncthreads();
  if (tid == 0) sm.bc[5] = add_acq_rel(P.seqctr + b, 1);
  __syncthreads();
  if (sm.bc[5] != K1 - 1) return;
  fence_acquire();
  if (GREEDY) finish_greedy(P, b);
  else finish_sampling<DT>(P, b, sm);
  __syncthreads();
  // the sequence's group records and tile masses have been consumed: clear them
  {
    uint32_t *gz = (uint32_t *)(P.grec + (int64_t)b * K1);
    const int ng = K1 * (int)(sizeof(GroupRec) / 4);
    for (int a = tid; a < ng; a += TPB) gz[a] = 0;
    if (!GREEDY) {
      double *rz = P.rsum + (int64_t)b * K1 * nT;
      for (int a = tid; a < K1 * nT; a += TPB) rz[a] = 0.0;
    }
  }
  if (tid == 0) st_relaxed(P.seqctr + b, 0);
  __syncthreads();
}

template <int DT, bool GREEDY>
__global__ __launch_bounds__(TPB) void spec_verify_kernel(Params P) {
  __shared__ Smem sm;
  for (int item = blockIdx.x; item < P.items; item += gridDim.x) {
    process_item<DT, GREEDY>(P, item, sm);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t sync, seqctr, fault, recs, rsum, grec, cand, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout_for(int B, int k, int V) {
  const size_t groups = (size_t)B * (k + 1);
  const size_t nT = ((size_t)V + TILE - 1) / TILE;
  Layout L;
  size_t o = 0;
  L.fault = o;  o = align256(o + sizeof(int32_t));      // fixed header, same offset for every shape
  L.sync = o;   o = align256(o + groups * sizeof(GroupSync));
  L.seqctr = o; o = align256(o + (size_t)B * sizeof(int32_t));
  L.recs = o;   o = align256(o + groups * nT * sizeof(TileRec));
  L.rsum = o;   o = align256(o + groups * nT * sizeof(double));
  L.grec = o;   o = align256(o + groups * sizeof(GroupRec));
  L.cand = o;   o = align256(o + groups * (size_t)(V < CAP ? V : CAP) * sizeof(uint64_t));
  L.total = o;
  return L;
}

struct DeviceInfo {
  bool ready = false;
  int cus = 0, coop = 0;
  int occ[4] = {0, 0, 0, 0};
};
std::mutex g_mu;
DeviceInfo g_dev[64];

typedef void (*kernel_fn)(Params);
kernel_fn kernel_for(int dtype, bool greedy) {
  if (dtype == SV_BF16) return greedy ? spec_verify_kernel<SV_BF16, true> : spec_verify_kernel<SV_BF16, false>;
  return greedy ? spec_verify_kernel<SV_F32, true> : spec_verify_kernel<SV_F32, false>;
}

int device_info(DeviceInfo *&out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo &d = g_dev[dev];
  if (!d.ready) {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return SV_ERR_HIP;
    if (hipDeviceGetAttribute(&d.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) return SV_ERR_HIP;
    for (int v = 0; v < 4; ++v) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void *)kernel_for(v >> 1, v & 1), TPB, 0) !=
          hipSuccess)
        return SV_ERR_HIP;
      d.occ[v] = nb;
    }
    d.ready = true;
  }
  out = &d;
  return SV_OK;
}

}  // namespace

extern "C" size_t spec_verify_workspace_bytes(const sv_shape_t *s) {
  if (!s || s->B < 0 || s->k < 0 || s->V < 1 || s->V > MAX_TILES * TILE) return 0;
  return layout_for(s->B, s->k, s->V).total;
}

extern "C" const char *spec_verify_error_string(int code) {
  switch (code) {
    case SV_OK: return "success";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "invalid shape (B<0, k<0, V<1, V>1048576, row stride < V, or sizes too large)";
    case SV_ERR_TEMPERATURE: return "temperature must be finite and >= 0";
    case SV_ERR_DTYPE: return "dtype must be SV_F32 or SV_BF16";
    case SV_ERR_WORKSPACE: return "workspace missing or smaller than spec_verify_workspace_bytes";
    case SV_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case SV_ERR_DEVICE: return "current device does not support cooperative launch";
    default: return "unknown error code";
  }
}

extern "C" int spec_verify(const sv_shape_t *shape, const void *target_logits, const void *draft_logits,
                           const int32_t *draft_tokens, const float *uniforms, int32_t *accepted_len,
                           int32_t *out_tokens, float *topk_val, int32_t *topk_idx, const sv_aux_t *aux,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (!shape) return SV_ERR_NULL;
  const sv_shape_t s = *shape;
  if (s.dtype != SV_F32 && s.dtype != SV_BF16) return SV_ERR_DTYPE;
  if (s.B < 0 || s.k < 0 || s.V < 1 || s.V > MAX_TILES * TILE) return SV_ERR_SHAPE;
  const int64_t ts = s.target_row_stride ? s.target_row_stride : s.V;
  const int64_t ds = s.draft_row_stride ? s.draft_row_stride : s.V;
  if (ts < s.V || ds < s.V) return SV_ERR_SHAPE;
  const int64_t nT = ((int64_t)s.V + TILE - 1) / TILE;
  const int64_t items = (int64_t)s.B * (s.k + 1) * nT;
  if (items > 0x7fffffffLL || (int64_t)s.B * (s.k + 2) > 0x7fffffffLL) return SV_ERR_SHAPE;
  if (!(s.temperature >= 0.f) || s.temperature == __builtin_inff()) return SV_ERR_TEMPERATURE;
  const bool greedy = s.temperature == 0.f;
  if (s.B == 0) return SV_OK;
  if (!target_logits || !accepted_len || !out_tokens || !topk_val || !topk_idx) return SV_ERR_NULL;
  if (s.k > 0 && !draft_tokens) return SV_ERR_NULL;
  if (!greedy && ((s.k > 0 && !draft_logits) || !uniforms)) return SV_ERR_NULL;
  const Layout L = layout_for(s.B, s.k, s.V);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;

  DeviceInfo *dev = nullptr;
  int rc = device_info(dev);
  if (rc != SV_OK) return rc;
  if (!dev->coop) return SV_ERR_DEVICE;

  char *ws = (char *)workspace;
  Params P;
  const int esz = s.dtype == SV_BF16 ? 2 : 4;
  P.target = (const char *)target_logits;
  P.draft = (const char *)draft_logits;
  P.tstride = ts;
  P.dstride = ds;
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.accepted_len = accepted_len;
  P.out_tokens = out_tokens;
  P.topk_val = topk_val;
  P.topk_idx = topk_idx;
  P.status = aux ? aux->status : nullptr;
  P.lse_t = aux ? aux->lse_target : nullptr;
  P.lse_d = aux ? aux->lse_draft : nullptr;
  P.p_tok = aux ? aux->p_tok : nullptr;
  P.q_tok = aux ? aux->q_tok : nullptr;
  P.sync = (GroupSync *)(ws + L.sync);
  P.seqctr = (int32_t *)(ws + L.seqctr);
  P.fault = (int32_t *)(ws + L.fault);
  P.recs = (TileRec *)(ws + L.recs);
  P.rsum = (double *)(ws + L.rsum);
  P.grec = (GroupRec *)(ws + L.grec);
  P.cand = (uint64_t *)(ws + L.cand);
  P.B = s.B;
  P.k = s.k;
  P.V = s.V;
  P.nT = (int32_t)nT;
  P.items = (int32_t)items;
  P.cap = s.V < CAP ? s.V : CAP;
  P.T = greedy ? 0.f : s.temperature;
  P.scd = greedy ? 0.0 : 1.4426950408889634 / (double)s.temperature;
  P.sc = (float)P.scd;
  P.t_vec = (((uintptr_t)target_logits & 15) == 0 && ((ts * esz) & 15) == 0) ? 1 : 0;
  P.d_vec = (!greedy && s.k > 0 && ((uintptr_t)draft_logits & 15) == 0 && ((ds * esz) & 15) == 0) ? 1 : 0;

  const int variant = (s.dtype == SV_BF16 ? 2 : 0) + (greedy ? 1 : 0);
  int64_t grid = (int64_t)dev->occ[variant] * dev->cus;
  if (const char *lim = getenv("SV_GRID_LIMIT")) {
    const long v = strtol(lim, nullptr, 10);
    if (v > 0 && v < grid) grid = v;
  }
  if (grid < nT) grid = nT;                      // a group must fit on the device at once
  if (grid > (int64_t)dev->occ[variant] * dev->cus) return SV_ERR_DEVICE;
  if (grid > items) grid = items;

  void *args[] = {&P};
  hipError_t e = hipLaunchCooperativeKernel((const void *)kernel_for(s.dtype, greedy), dim3((unsigned)grid),
                                            dim3(TPB), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return SV_ERR_HIP;
  }
  return SV_OK;
}
