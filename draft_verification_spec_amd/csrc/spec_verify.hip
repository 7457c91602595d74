// spec_verify.hip -- speculative-sampling verification for gfx950 (MI355X).
//
// Two plain launches and no waiting between workgroups:
//
//  sv_stream  one workgroup per (group, tile).  A "group" is, for i < k, the
//             pair (target row i, draft row i) of a sequence; group k is target
//             row k alone; in greedy mode every group is one target row.  Tiles
//             are fixed vocabulary slices (4096 entries for bf16, 2048 for fp32:
//             8 KB per row either way).  Each workgroup streams its tile(s) once
//             with 128-bit loads and publishes:
//               - per-row-part max and sum of exp2((x - max) * log2(e)/T)
//                 (fp32 exp, per-thread fp32 sums, fp64 above the thread);
//               - the target tile's top-32 candidates: every element at or above
//                 the tile's 32nd largest lane maximum (at least 32 elements of
//                 the tile lie there, so the tile's top-32 is among them).
//             The last workgroup of a group to publish combines the tile records
//             in tile order into the row max and normaliser, takes the row's
//             acceptance decision, and merges the candidates that reach the row
//             bound (the largest tile bound) into the top-32 (value desc, index
//             asc).  The last group of a sequence finds the first rejection j
//             (or emits the greedy argmax-prefix result).
//  sv_draw    sampling only: one workgroup per tile of the drawing row (row j's
//             pair for a rejection, target row k after k acceptances) publishes
//             the tile's residual mass max(0, p - q) (or p); the last one draws
//             by inverse CDF over the tile masses in tile order and rescans the
//             crossing tile element by element.
//
// Cross-workgroup data within a launch moves through the workspace with
// device-scope write-through stores and device-scope loads, ordered by waiting
// for the stores to complete before the counter that announces them is bumped.
// No workgroup ever waits for another, so any launch order and any occupancy
// are safe.
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

#include "spec_verify.h"

namespace {

constexpr int TPB = 256;               // threads per workgroup (4 waves of 64)
constexpr int NWAVE = TPB / 64;
constexpr int NSEG = 2;                // 16-byte vectors per thread per row
constexpr int SLOTS = 64;              // candidate slots per tile
constexpr int MERGE_CAP = 512;         // candidates a row merge ranks in LDS
constexpr int TOPK = SV_TOPK;
constexpr int MAX_TILES = 128;
constexpr float NEG_INF = -__builtin_inff();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Fmt;
template <> struct Fmt<SV_BF16> { static constexpr int E = 2, W = 8, TILE = TPB * NSEG * 8; };
template <> struct Fmt<SV_F32> { static constexpr int E = 4, W = 4, TILE = TPB * NSEG * 4; };

// Published per (group, tile) by sv_stream.
struct TileRec {
  float m_t, m_d;          // tile max of the target / draft row part
  double s_t, s_d;         // sum exp2((x - m) * sc) over the tile part
  uint32_t bound;          // ordered key of the tile's 32nd largest lane maximum (0: fewer lanes)
  int32_t flags_t, flags_d;
  int32_t overflow;        // more candidates than SLOTS
  uint32_t top[4];         // ordered keys of the tile's 4 largest lane maxima (0: no lane)
  int32_t pad[2];
};

// Published per group by its last workgroup.
struct GroupRec {
  double s_t, s_d;         // row normalisers (relative to m_t, m_d)
  float m_t, m_d;          // row maxima
  int32_t flags;           // SV_STATUS_* bits of this group's rows and token
  int32_t accept;          // 1 when the drafted token passed (pair groups)
  int32_t argmax;          // top-1 index of the target row
  int32_t pad;
};

// Handed from sv_stream to sv_draw per sequence (valid == 1: a token to draw).
struct SeqRec {
  double s_t, s_d;         // normalisers of the drawing row's target / draft part
  float m_t, m_d;
  int32_t j, valid;        // drawing position, and whether sv_draw has work
  double u;                // the uniform of the draw
  int32_t resid, pad;      // 1: residual of the pair row j; 0: target row k
};

struct Params {
  const char *target, *draft;
  int64_t tstride, dstride;            // row strides in elements
  const int32_t *tokens;
  const float *uniforms;
  int32_t *accepted_len, *out_tokens, *topk_idx, *status;
  float *topk_val, *lse_t, *lse_d, *p_tok, *q_tok;
  int32_t *fault;                      // set when the workspace was not zero-filled
  int32_t *garrive, *sarrive, *darrive;
  TileRec *recs;
  GroupRec *grec;
  SeqRec *srec;
  uint64_t *cand;                      // [group][tile][SLOTS] candidate keys, 0 = empty
  double *rsum;                        // [sequence][tile] masses of the drawing row
  int32_t B, k, V, nT;
  float T, sc;                         // sc = log2(e) / T
  double scd;
  int32_t t_vec, d_vec;                // rows 16-byte aligned
};

struct Smem {
  union {
    uint32_t lists[NWAVE][32];         // per-wave top-32 lane maxima
    uint32_t tops[4 * MAX_TILES];      // row merge: the tiles' largest lane maxima
    uint64_t keys[MERGE_CAP];          // row merge: candidate keys
    struct {                           // exact top-32 fallback
      uint32_t hist[2048];
      int32_t part[TPB];
      uint64_t list[TOPK];
    } fb;
    double tot[MAX_TILES];             // draw: tile masses
  };
  float f[4][NWAVE];
  uint32_t u[2][NWAVE];
  int32_t i[4][NWAVE];
  double d[4][NWAVE];
  int32_t bc[8];
  double dbc[4];
  uint64_t ovmask[NWAVE];              // row merge: tiles whose candidates overflowed
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
// 64-bit candidate key, larger = earlier in (value desc, index asc): the
// ordered value above, the complemented index (V <= 2^20) and a -0.0 marker
// in the lowest bit (it never decides an order: indices differ by >= 1).
__device__ __forceinline__ uint64_t cand_key(float v, int32_t x) {
  const uint32_t neg0 = __float_as_uint(v) == 0x80000000u ? 1u : 0u;
  return ((uint64_t)ordered_key(v) << 32) | ((uint64_t)(0xfffffu - (uint32_t)x) << 1) | neg0;
}
__device__ __forceinline__ int32_t cand_index(uint64_t k) { return (int32_t)(0xfffffu - ((uint32_t)k >> 1)); }
__device__ __forceinline__ float cand_value(uint64_t k) {
  return (k & 1u) ? -0.0f : key_value((uint32_t)(k >> 32));
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
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { int w = __shfl_xor(v, o); v = w < v ? w : v; }
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
// Bitonic sort of one value per lane, descending across the wave's 64 lanes.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t o = __shfl_xor(v, j);
      const bool desc = (lane & k) == 0, lower = (lane & j) == 0;
      const uint32_t hi = v > o ? v : o, lo = v > o ? o : v;
      v = (lower == desc) ? hi : lo;
    }
  }
  return v;
}

// Device-scope accesses: loads see the latest device-visible value; stores are
// written through to the device coherence point.  No cache maintenance.
template <class T> __device__ __forceinline__ T ld_dev(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T> __device__ __forceinline__ void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_dev(int32_t *p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's earlier memory accesses have completed (and keep the
// compiler from moving memory accesses across the wait).
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
// Announce this workgroup's published data on a counter; returns the count
// before it (the same value in every thread).
__device__ __forceinline__ int arrive(int32_t *ctr, Smem &sm) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) sm.bc[7] = add_dev(ctr, 1);
  __syncthreads();
  const int old = sm.bc[7];
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return old;
}
// Records move as 64-bit words.
template <class T> __device__ __forceinline__ void st_rec(T *dst, const T &v) {
  static_assert(sizeof(T) % 8 == 0, "record size");
  const uint64_t *s = (const uint64_t *)&v;
  uint64_t *d = (uint64_t *)dst;
#pragma unroll
  for (int w = 0; w < (int)(sizeof(T) / 8); ++w) st_dev(d + w, s[w]);
}
template <class T> __device__ __forceinline__ T ld_rec(const T *src) {
  static_assert(sizeof(T) % 8 == 0, "record size");
  T v;
  uint64_t *d = (uint64_t *)&v;
  const uint64_t *s = (const uint64_t *)src;
#pragma unroll
  for (int w = 0; w < (int)(sizeof(T) / 8); ++w) d[w] = ld_dev(s + w);
  return v;
}
template <class T> __device__ __forceinline__ void zero_recs(T *dst, int n) {
  uint64_t *d = (uint64_t *)dst;
  const int words = n * (int)(sizeof(T) / 8);
  for (int w = threadIdx.x; w < words; w += TPB) st_dev(d + w, (uint64_t)0);
}

template <int DT> __device__ __forceinline__ float load_elem(const char *row, int64_t x) {
  if constexpr (DT == SV_BF16) {
    return __uint_as_float((uint32_t)(*(const uint16_t *)(row + x * 2)) << 16);
  } else {
    return *(const float *)(row + x * 4);
  }
}

// element w of a 16-byte vector
template <int DT> __device__ __forceinline__ float unpack(const u32x4 &v, int w) {
  if constexpr (DT == SV_BF16) {
    const uint32_t word = v[w >> 1];
    return __uint_as_float((w & 1) ? (word & 0xffff0000u) : (word << 16));
  } else {
    return __uint_as_float(v[w]);
  }
}

// tile-local position of element w of this thread's vector s
template <int DT> __device__ __forceinline__ int tpos(int s, int w) {
  return s * (TPB * Fmt<DT>::W) + (int)threadIdx.x * Fmt<DT>::W + w;
}

// Stream one tile of a row into registers; entries past V read as -inf.
template <int DT>
__device__ __forceinline__ void load_tile(const char *row, int c, int V, bool vec, u32x4 (&r)[NSEG]) {
  constexpr int E = Fmt<DT>::E, W = Fmt<DT>::W;
  const int64_t c0 = (int64_t)c * Fmt<DT>::TILE;
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

template <int DT> __device__ __forceinline__ float thread_max(const u32x4 (&r)[NSEG]) {
  float m = NEG_INF;
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) m = fmaxf(m, unpack<DT>(r[s], w));
  return m;
}

template <int DT> __device__ __forceinline__ bool thread_has_nan(const u32x4 (&r)[NSEG]) {
  bool nan = false;
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) { const float x = unpack<DT>(r[s], w); nan |= !(x == x); }
  return nan;
}

// exp2((x - m) * sc) of one element; a thread whose slice is all -inf uses 0 as m
__device__ __forceinline__ float scaled_exp(float x, float m, float sc) {
  const float ms = (m == NEG_INF) ? 0.f : m;
  return __builtin_amdgcn_exp2f((x - ms) * sc);
}

// Sequential fp32 sum of the thread's scaled exps; flags NaN / +inf.
template <int DT>
__device__ __forceinline__ float thread_expsum(const u32x4 (&r)[NSEG], float m, float sc, int &flags) {
  float s = 0.f;
#pragma unroll
  for (int g = 0; g < NSEG; ++g)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) s += scaled_exp(unpack<DT>(r[g], w), m, sc);
  flags = 0;
  if (!(s == s)) flags = thread_has_nan<DT>(r) ? SV_STATUS_NAN : SV_STATUS_POSINF;
  return s;
}

// Per-thread scale turning scaled exps into probabilities: exp2((m_thread - m_row) * sc) / s_row.
__device__ __forceinline__ float prob_scale(float m_thr, float m_row, double s_row, float sc) {
  if (m_thr == NEG_INF) return 0.f;
  return (float)((double)__builtin_amdgcn_exp2f((m_thr - m_row) * sc) / s_row);
}

// Mass of one element: residual max(0, p - q) for a pair row, p for a single row.
template <int DT>
__device__ __forceinline__ float elem_mass(const u32x4 &vt, const u32x4 &vd, int w, bool resid, float mt, float md,
                                           float at, float ad, float sc) {
  const float p = scaled_exp(unpack<DT>(vt, w), mt, sc) * at;
  if (!resid) return p;
  const float q = scaled_exp(unpack<DT>(vd, w), md, sc) * ad;
  const float r = p - q;
  return r > 0.f ? r : 0.f;
}

// Sequential fp32 mass of each of the thread's vectors.
template <int DT>
__device__ __forceinline__ void seg_masses(const u32x4 (&rt)[NSEG], const u32x4 (&rd)[NSEG], bool resid, float mt,
                                           float md, float at, float ad, float sc, float (&seg)[NSEG]) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) a += elem_mass<DT>(rt[s], rd[s], w, resid, mt, md, at, ad, sc);
    seg[s] = a;
  }
}

// Exclusive prefix (fp64) of per-thread vector masses over the tile, in the
// tile's element order (vector-major, then thread).  base[s] receives the mass
// of all tile elements before this thread's vector s; returns the tile total.
// Fixed association: identical bits wherever it is evaluated.
__device__ double tile_scan(const float (&seg)[NSEG], double (&base)[NSEG], Smem &sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  double acc = 0.0;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const double x = (double)seg[s];
    const double inc = wave_incl_dbl(x, lane);
    double prev = __shfl_up(inc, 1);
    if (lane == 0) prev = 0.0;
    if (lane == 63) sm.d[s][wid] = inc;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wid; ++w) off += sm.d[s][w];
    double tot = 0.0;
    for (int w = 0; w < NWAVE; ++w) tot += sm.d[s][w];
    base[s] = acc + (off + prev);
    acc = acc + tot;
  }
  __syncthreads();
  return acc;
}

// Block-wide OR and MIN through LDS.
__device__ __forceinline__ void block_or_min(int &o, int &m, Smem &sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  o = wave_or(o);
  m = wave_min_i(m);
  if (lane == 0) { sm.i[0][wid] = o; sm.i[1][wid] = m; }
  __syncthreads();
  o = sm.i[0][0];
  m = sm.i[1][0];
  for (int w = 1; w < NWAVE; ++w) { o |= sm.i[0][w]; m = sm.i[1][w] < m ? sm.i[1][w] : m; }
  __syncthreads();
}

// Top-32 of a target row by exact radix selection over the whole row (used
// when the candidate slots overflowed).  Rank 0's index goes to sm.bc[6].
template <int DT>
__device__ void topk_exact(const char *row, int V, float *oval, int32_t *oidx, Smem &sm) {
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
    float v = 0.f;
    uint32_t key = 0;
    if (x < V) { v = load_elem<DT>(row, x); key = ordered_key(v); }
    if (x < V && key > theta) {
      const int slot = atomicAdd(&sm.bc[2], 1);
      sm.fb.list[slot] = cand_key(v, x);
    }
    const bool eq = x < V && key == theta;
    const uint64_t bal = __ballot(eq);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sm.i[0][wid] = __popcll(bal);
    __syncthreads();
    int woff = sm.bc[3];
    for (int w = 0; w < wid; ++w) woff += sm.i[0][w];
    const int rank = woff + before;
    if (eq && rank < eq_need) sm.fb.list[above + rank] = cand_key(v, x);
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
    oidx[rank] = cand_index(ka);
    oval[rank] = cand_value(ka);
    if (rank == 0) sm.bc[6] = cand_index(ka);
  }
  for (int r = need + tid; r < TOPK; r += TPB) { oidx[r] = -1; oval[r] = NEG_INF; }
  __syncthreads();
}

struct Geo {
  int g, c, b, i;
  bool pair;
  const char *trow, *drow;
};

template <int DT, bool GREEDY> __device__ __forceinline__ Geo geo(const Params &P, int item) {
  Geo G;
  const int K1 = P.k + 1;
  G.g = item / P.nT;
  G.c = item - G.g * P.nT;
  G.b = G.g / K1;
  G.i = G.g - G.b * K1;
  G.pair = !GREEDY && G.i < P.k;
  G.trow = P.target + ((int64_t)G.b * K1 + G.i) * P.tstride * Fmt<DT>::E;
  G.drow = G.pair ? P.draft + ((int64_t)G.b * P.k + G.i) * P.dstride * Fmt<DT>::E : nullptr;
  return G;
}

// Row combine, acceptance decision and top-32 merge of group g (run by the
// last workgroup of the group to publish).
template <int DT, bool GREEDY>
__device__ void group_finish(const Params &P, const Geo &G, Smem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1, V = P.V;
  const int g = G.g, b = G.b, i = G.i;
  const bool pair = G.pair;
  // the tile records (nT <= TPB: thread cc holds tile cc) and the drafted token's logits
  TileRec rec;
  const bool own = tid < nT;
  if (own) {
    rec = ld_rec(P.recs + (int64_t)g * nT + tid);
  } else {
    rec.m_t = NEG_INF; rec.m_d = NEG_INF; rec.s_t = 0.0; rec.s_d = 0.0;
    rec.bound = 0; rec.flags_t = 0; rec.flags_d = 0; rec.overflow = 0;
    for (int w = 0; w < 4; ++w) rec.top[w] = 0;
  }
  if (own)
    for (int w = 0; w < 4; ++w) sm.tops[tid * 4 + w] = rec.top[w];
  int32_t x = -1;
  float tx = 0.f, dx = 0.f;
  if (pair && tid == 0) {
    x = P.tokens[(int64_t)b * k + i];
    if (x >= 0 && x < V) { tx = load_elem<DT>(G.trow, x); dx = load_elem<DT>(G.drow, x); }
  }
  {
    const float a = wave_max(rec.m_t), d = wave_max(rec.m_d);
    const int fa = wave_or(rec.flags_t), fb = wave_or(rec.flags_d);
    const uint32_t bd = wave_max_u(rec.bound);
    const uint64_t ov = __ballot(own && rec.overflow);
    if (lane == 0) {
      sm.f[2][wid] = a; sm.f[3][wid] = d; sm.i[2][wid] = fa; sm.i[3][wid] = fb; sm.u[1][wid] = bd;
      sm.ovmask[wid] = ov;
    }
  }
  __syncthreads();
  float m_rt = sm.f[2][0], m_rd = sm.f[3][0];
  int f_rt = sm.i[2][0], f_rd = sm.i[3][0];
  uint32_t L = sm.u[1][0];
  for (int w = 1; w < NWAVE; ++w) {
    m_rt = fmaxf(m_rt, sm.f[2][w]); m_rd = fmaxf(m_rd, sm.f[3][w]);
    f_rt |= sm.i[2][w]; f_rd |= sm.i[3][w];
    L = sm.u[1][w] > L ? sm.u[1][w] : L;
  }
  double s_rt = 0.0, s_rd = 0.0;
  if (!GREEDY) {
    double a = 0.0, d = 0.0;
    if (own && rec.m_t != NEG_INF) a = rec.s_t * (double)__builtin_amdgcn_exp2f((rec.m_t - m_rt) * P.sc);
    if (own && pair && rec.m_d != NEG_INF) d = rec.s_d * (double)__builtin_amdgcn_exp2f((rec.m_d - m_rd) * P.sc);
    a = wave_sum(a);
    d = wave_sum(d);
    if (lane == 0) { sm.d[2][wid] = a; sm.d[3][wid] = d; }
    __syncthreads();
    for (int w = 0; w < NWAVE; ++w) { s_rt += sm.d[2][w]; s_rd += sm.d[3][w]; }
  }
  // one data-error bit per row: NaN before +inf before an empty row
  f_rt = (f_rt & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rt;
  f_rd = (f_rd & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rd;
  if (!GREEDY && m_rt == NEG_INF && !f_rt) f_rt = SV_STATUS_EMPTY_ROW;
  if (pair && m_rd == NEG_INF && !f_rd) f_rd = SV_STATUS_EMPTY_ROW;

  // A tighter row bound: the 32nd largest of the tiles' 4 largest lane maxima
  // (32 distinct lanes hold an element at or above it).  The row's 32nd
  // largest element is at or above both bounds, and every element at or above
  // L sits in its tile's slots.
  if (wid == 0) {
    const int nkeys = nT * 4;
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int cnt = 0;
      for (int j0 = 0; j0 < nkeys; j0 += 64) {
        const int jj = j0 + lane;
        cnt += __popcll(__ballot(jj < nkeys && sm.tops[jj] >= cand));
      }
      if (cnt >= TOPK) prefix = cand;
    }
    if (lane == 0) sm.u[0][0] = prefix;
  }
  __syncthreads();
  L = sm.u[0][0] > L ? sm.u[0][0] : L;
  // candidates reaching the row bound; every non-empty slot is cleared.  A tile
  // that had more candidates than slots is rescanned here against the bound.
  if (tid == 0) { sm.bc[0] = 0; sm.bc[6] = -1; }
  __syncthreads();
  uint64_t *slots = P.cand + (int64_t)g * nT * SLOTS;
  for (int a = tid; a < nT * SLOTS; a += TPB) {
    const uint64_t key = ld_dev(slots + a);
    if (key) {
      st_dev(slots + a, (uint64_t)0);
      const int tc = a / SLOTS;
      const bool ovf = (sm.ovmask[tc >> 6] >> (tc & 63)) & 1u;
      if (!ovf && (uint32_t)(key >> 32) >= L) {
        const int pos = atomicAdd(&sm.bc[0], 1);
        if (pos < MERGE_CAP) sm.keys[pos] = key;
      }
    }
  }
  for (int wq = 0; wq < NWAVE; ++wq) {
    uint64_t m = sm.ovmask[wq];
    while (m) {
      const int tc = wq * 64 + __builtin_ctzll(m);
      m &= m - 1;
      u32x4 r[NSEG];
      load_tile<DT>(G.trow, tc, V, P.t_vec, r);
      const int lim = V - tc * Fmt<DT>::TILE;
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int w = 0; w < Fmt<DT>::W; ++w) {
          const float xv = unpack<DT>(r[s], w);
          if (tpos<DT>(s, w) < lim && xv == xv && ordered_key(xv) >= L) {
            const int pos = atomicAdd(&sm.bc[0], 1);
            if (pos < MERGE_CAP) sm.keys[pos] = cand_key(xv, tc * Fmt<DT>::TILE + tpos<DT>(s, w));
          }
        }
    }
  }
  __syncthreads();
  const int n = sm.bc[0];
  const bool overflow = false;
  float *oval = P.topk_val + ((int64_t)b * K1 + i) * TOPK;
  int32_t *oidx = P.topk_idx + ((int64_t)b * K1 + i) * TOPK;
  if (f_rt & SV_STATUS_NAN) {
    for (int r = tid; r < TOPK; r += TPB) { oval[r] = __builtin_nanf(""); oidx[r] = -1; }
  } else if (overflow || n > MERGE_CAP) {
    topk_exact<DT>(G.trow, V, oval, oidx, sm);
  } else {
    for (int a = tid; a < n; a += TPB) {
      const uint64_t ka = sm.keys[a];
      int rank = 0;
      for (int jj = 0; jj < n; ++jj) rank += sm.keys[jj] > ka;
      if (rank < TOPK) {
        oidx[rank] = cand_index(ka);
        oval[rank] = cand_value(ka);
        if (rank == 0) sm.bc[6] = cand_index(ka);
      }
    }
    for (int r = n + tid; r < TOPK; r += TPB) { oval[r] = NEG_INF; oidx[r] = -1; }
  }
  __syncthreads();

  // acceptance decision of the row; the group record for the sequence
  if (tid == 0) {
    int fl = GREEDY ? (f_rt & SV_STATUS_NAN) : (f_rt | (pair ? f_rd : 0));
    int acc = 1;
    float pt = __builtin_nanf(""), qt = __builtin_nanf("");
    if (pair) {
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
    }
    GroupRec gr;
    gr.s_t = s_rt; gr.s_d = s_rd; gr.m_t = m_rt; gr.m_d = m_rd;
    gr.flags = fl; gr.accept = acc; gr.argmax = sm.bc[6]; gr.pad = 0;
    st_rec(P.grec + g, gr);
    if (!GREEDY) {
      if (P.lse_t) P.lse_t[(int64_t)b * K1 + i] = (float)((double)m_rt / (double)P.T + log(s_rt));
      if (pair) {
        if (P.p_tok) P.p_tok[(int64_t)b * k + i] = pt;
        if (P.q_tok) P.q_tok[(int64_t)b * k + i] = qt;
        if (P.lse_d) P.lse_d[(int64_t)b * k + i] = (float)((double)m_rd / (double)P.T + log(s_rd));
      }
    }
  }
  // every workgroup of the group has published and left: clear the group
  zero_recs(P.recs + (int64_t)g * nT, nT);
  if (tid == 0) st_dev(P.garrive + g, 0);
}

// Sequence assembly in sv_stream (run by the last group of the sequence):
// greedy emits everything; sampling emits all but the drawn token and hands
// the drawing row to sv_draw.
template <bool GREEDY>
__device__ void seq_finish(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1;
  int st = 0, j = k;
  for (int i = tid; i <= k; i += TPB) {
    const GroupRec r = ld_rec(P.grec + (int64_t)b * K1 + i);
    st |= r.flags;
    if (i < k) {
      if (GREEDY) {
        const int32_t x = P.tokens[(int64_t)b * k + i];
        if (x < 0 || x >= P.V) st |= SV_STATUS_BAD_TOKEN;
        else if (x != r.argmax && i < j) j = i;
      } else if (!r.accept && i < j) {
        j = i;
      }
    }
  }
  if (!GREEDY)
    for (int i = tid; i < k + 2; i += TPB) {
      const float u = P.uniforms[(int64_t)b * (k + 2) + i];
      if (!(u >= 0.f && u < 1.f)) st |= SV_STATUS_BAD_UNIFORM;
    }
  if (tid == 0 && ld_dev(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
  block_or_min(st, j, sm);
  if (tid == 0) {
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
    const GroupRec rj = ld_rec(P.grec + (int64_t)b * K1 + j);
    if (GREEDY) {
      sm.bc[1] = rj.argmax;
    } else if (!st) {
      SeqRec sr;
      sr.s_t = rj.s_t; sr.s_d = rj.s_d; sr.m_t = rj.m_t; sr.m_d = rj.m_d;
      sr.j = j; sr.valid = 1;
      sr.u = (double)P.uniforms[(int64_t)b * (k + 2) + (j < k ? k : k + 1)];
      sr.resid = j < k ? 1 : 0; sr.pad = 0;
      P.srec[b] = sr;                  // read by sv_draw after this launch
    }
  }
  __syncthreads();
  for (int i = tid; i < K1; i += TPB) {
    int v = -1;
    if (!st && i < j) v = P.tokens[(int64_t)b * k + i];
    if (!st && i == j && GREEDY) v = sm.bc[1];
    if (st || i != j || GREEDY) P.out_tokens[(int64_t)b * K1 + i] = v;
  }
  __syncthreads();
  zero_recs(P.grec + (int64_t)b * K1, K1);
  if (tid == 0) st_dev(P.sarrive + b, 0);
}

template <int DT, bool GREEDY>
__global__ __launch_bounds__(TPB) void sv_stream(Params P) {
  __shared__ Smem sm;
  constexpr int W = Fmt<DT>::W, TILE = Fmt<DT>::TILE;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, V = P.V;
  const int item = blockIdx.x;
  const Geo G = geo<DT, GREEDY>(P, item);
  const int g = G.g, c = G.c;
  const bool pair = G.pair;

  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(G.trow, c, V, P.t_vec, rt);
  if (pair) load_tile<DT>(G.drow, c, V, P.d_vec, rd);
  else
#pragma unroll
    for (int s = 0; s < NSEG; ++s) rd[s] = rt[s];

  // per-thread statistics
  const float mt = thread_max<DT>(rt);
  const float md = pair ? thread_max<DT>(rd) : NEG_INF;
  int ft = 0, fd = 0;
  float st = 0.f, sd = 0.f;
  if (!GREEDY) {
    st = thread_expsum<DT>(rt, mt, P.sc, ft);
    if (pair) sd = thread_expsum<DT>(rd, md, P.sc, fd);
  } else {
    ft = thread_has_nan<DT>(rt) ? SV_STATUS_NAN : 0;
  }
  const bool has_elem = (int64_t)c * TILE + (int64_t)tid * W < V;
  const uint32_t tkey = has_elem ? ordered_key(mt) : 0u;

  // per-wave top-32 lane maxima, tile max and flags
  const uint32_t sorted = wave_sort_desc(tkey, lane);
  if (lane < 32) sm.lists[wid][lane] = sorted;
  {
    const float wm_t = wave_max(mt), wm_d = wave_max(md);
    const int wf_t = wave_or(ft), wf_d = wave_or(fd);
    if (lane == 0) { sm.f[0][wid] = wm_t; sm.f[1][wid] = wm_d; sm.i[0][wid] = wf_t; sm.i[1][wid] = wf_d; }
  }
  __syncthreads();
  // the tile bound: 32nd largest of the 256 lane maxima (top 32 of each pair
  // of sorted lists merged, then sorted)
  if (wid == 0) {
    const int h = lane & 31;
    const uint32_t p = lane < 32 ? sm.lists[0][h] : sm.lists[2][h];
    const uint32_t q = lane < 32 ? sm.lists[1][31 - h] : sm.lists[3][31 - h];
    const uint32_t s2 = wave_sort_desc(p > q ? p : q, lane);
    const uint32_t b32 = __shfl(s2, 31);
    if (lane == 0) sm.u[0][0] = b32;
    if (lane < 4) sm.u[1][lane] = s2;
  }
  float m_ct = sm.f[0][0], m_cd = sm.f[1][0];
  int f_ct = sm.i[0][0], f_cd = sm.i[1][0];
  for (int w = 1; w < NWAVE; ++w) {
    m_ct = fmaxf(m_ct, sm.f[0][w]); m_cd = fmaxf(m_cd, sm.f[1][w]);
    f_ct |= sm.i[0][w]; f_cd |= sm.i[1][w];
  }
  if (!GREEDY) {
    double a = (mt == NEG_INF) ? 0.0 : (double)st * (double)__builtin_amdgcn_exp2f((mt - m_ct) * P.sc);
    double d = 0.0;
    if (pair) d = (md == NEG_INF) ? 0.0 : (double)sd * (double)__builtin_amdgcn_exp2f((md - m_cd) * P.sc);
    a = wave_sum(a);
    d = wave_sum(d);
    if (lane == 0) { sm.d[0][wid] = a; sm.d[1][wid] = d; }
  }
  __syncthreads();
  double s_ct = 0.0, s_cd = 0.0;
  if (!GREEDY) for (int w = 0; w < NWAVE; ++w) { s_ct += sm.d[0][w]; s_cd += sm.d[1][w]; }
  const uint32_t bound = sm.u[0][0];

  // candidates: elements at or above the bound, to this tile's slots in element order
  int overflow = 0;
  {
    const float Lf = key_value(bound);
    const int lim = V - c * TILE;                        // tile positions < lim exist
    uint32_t mask = 0;
    if (has_elem && (bound == 0u || mt >= Lf)) {
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float xv = unpack<DT>(rt[s], w);
          if (tpos<DT>(s, w) < lim && (bound == 0u || xv >= Lf)) mask |= 1u << (s * W + w);
        }
    }
    const int cnt = __popc(mask);
    const int inc = wave_incl_int(cnt, lane);
    if (lane == 63) sm.i[2][wid] = inc;
    __syncthreads();
    int slot = inc - cnt, total = 0;
    for (int w = 0; w < NWAVE; ++w) { if (w < wid) slot += sm.i[2][w]; total += sm.i[2][w]; }
    uint64_t *dst = P.cand + ((int64_t)g * nT + c) * SLOTS;
    while (mask) {
      const int bit = __builtin_ctz(mask);
      mask &= mask - 1;
      const int s = bit / W, w = bit - s * W;
      if (slot < SLOTS) st_dev(dst + slot, cand_key(unpack<DT>(rt[s], w), c * TILE + tpos<DT>(s, w)));
      ++slot;
    }
    overflow = total > SLOTS ? 1 : 0;
  }

  if (tid == 0) {
    TileRec r;
    r.m_t = m_ct; r.m_d = m_cd; r.s_t = s_ct; r.s_d = s_cd;
    r.bound = bound; r.flags_t = f_ct; r.flags_d = f_cd; r.overflow = overflow;
    for (int w = 0; w < 4; ++w) r.top[w] = sm.u[1][w];
    r.pad[0] = 0; r.pad[1] = 0;
    st_rec(P.recs + item, r);
  }
  const int old = arrive(P.garrive + g, sm);
  if (old < 0 || old >= nT) { if (tid == 0) atomicOr(P.fault, 2); return; }  // workspace not zero-filled
  if (old != nT - 1) return;
  group_finish<DT, GREEDY>(P, G, sm);
  const int olds = arrive(P.sarrive + G.b, sm);
  if (olds != P.k) return;
  seq_finish<GREEDY>(P, G.b, sm);
}

// Inverse-CDF draw inside one tile: the first element (ascending index) of
// positive mass whose cumulative mass prefix + (scan base + running fp32 sum)
// exceeds tau; if rounding leaves none, the tile's last positive-mass element.
// The masses are recomputed exactly as when the tile's total was published.
template <int DT>
__device__ int tile_draw(const Params &P, const char *trow, const char *drow, int c, bool resid, float m_t,
                         double s_t, float m_d, double s_d, double prefix, double tau, Smem &sm) {
  constexpr int W = Fmt<DT>::W;
  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(trow, c, P.V, P.t_vec, rt);
  if (resid) load_tile<DT>(drow, c, P.V, P.d_vec, rd);
  else
#pragma unroll
    for (int s = 0; s < NSEG; ++s) rd[s] = rt[s];
  const float mt = thread_max<DT>(rt);
  const float md = resid ? thread_max<DT>(rd) : NEG_INF;
  const float at = prob_scale(mt, m_t, s_t, P.sc);
  const float ad = resid ? prob_scale(md, m_d, s_d, P.sc) : 0.f;
  float seg[NSEG];
  seg_masses<DT>(rt, rd, resid, mt, md, at, ad, P.sc, seg);
  double base[NSEG];
  tile_scan(seg, base, sm);
  int first = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mval = elem_mass<DT>(rt[s], rd[s], w, resid, mt, md, at, ad, P.sc);
      a += mval;
      const int pos = tpos<DT>(s, w);
      if (mval > 0.f) {
        lastpos = pos > lastpos ? pos : lastpos;
        if (prefix + (base[s] + (double)a) > tau && pos < first) first = pos;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const int f2 = __shfl_xor(first, o), l2 = __shfl_xor(lastpos, o);
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
  return pos < 0 ? -1 : c * Fmt<DT>::TILE + pos;
}

// Total target mass p of one tile (the arithmetic of tile_draw without a draft row).
template <int DT>
__device__ double tile_mass_p(const Params &P, const char *trow, int c, float m_t, double s_t, Smem &sm) {
  u32x4 rt[NSEG];
  load_tile<DT>(trow, c, P.V, P.t_vec, rt);
  const float mt = thread_max<DT>(rt);
  const float at = prob_scale(mt, m_t, s_t, P.sc);
  float seg[NSEG];
  seg_masses<DT>(rt, rt, false, mt, NEG_INF, at, 0.f, P.sc, seg);
  double base[NSEG];
  return tile_scan(seg, base, sm);
}

template <int DT>
__global__ __launch_bounds__(TPB) void sv_draw(Params P) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int nT = P.nT, k = P.k, K1 = k + 1;
  const int b = blockIdx.x / nT, c = blockIdx.x - (blockIdx.x / nT) * nT;
  const SeqRec sr = P.srec[b];
  if (!sr.valid) return;
  const int j = sr.j;
  const bool resid = sr.resid != 0;
  const char *trow = P.target + ((int64_t)b * K1 + j) * P.tstride * Fmt<DT>::E;
  const char *drow = resid ? P.draft + ((int64_t)b * k + j) * P.dstride * Fmt<DT>::E : nullptr;
  {
    u32x4 rt[NSEG], rd[NSEG];
    load_tile<DT>(trow, c, P.V, P.t_vec, rt);
    if (resid) load_tile<DT>(drow, c, P.V, P.d_vec, rd);
    else
#pragma unroll
      for (int s = 0; s < NSEG; ++s) rd[s] = rt[s];
    const float mt = thread_max<DT>(rt);
    const float md = resid ? thread_max<DT>(rd) : NEG_INF;
    const float at = prob_scale(mt, sr.m_t, sr.s_t, P.sc);
    const float ad = resid ? prob_scale(md, sr.m_d, sr.s_d, P.sc) : 0.f;
    float seg[NSEG];
    seg_masses<DT>(rt, rd, resid, mt, md, at, ad, P.sc, seg);
    double base[NSEG];
    const double tot = tile_scan(seg, base, sm);
    if (tid == 0) st_dev(P.rsum + (int64_t)b * nT + c, tot);
  }
  const int old = arrive(P.darrive + b, sm);
  if (old < 0 || old >= nT) { if (tid == 0) atomicOr(P.fault, 2); return; }
  if (old != nT - 1) return;

  // last tile of the row: locate the crossing tile in tile order, rescan it
  for (int cc = tid; cc < nT; cc += TPB) sm.tot[cc] = ld_dev(P.rsum + (int64_t)b * nT + cc);
  __syncthreads();
  bool use_p = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (tid == 0) {
      double R = 0.0;
      for (int cc = 0; cc < nT; ++cc) R += sm.tot[cc];
      const double tau = sr.u * R;
      double Pc = 0.0;
      int cs = -1;
      for (int cc = 0; cc < nT; ++cc) {
        const double nx = Pc + sm.tot[cc];
        if (nx > tau) { cs = cc; break; }
        Pc = nx;
      }
      sm.bc[2] = cs;
      sm.dbc[0] = Pc;
      sm.dbc[1] = tau;
    }
    __syncthreads();
    if (sm.bc[2] >= 0 || attempt == 1) break;
    // no residual mass left (only through rounding): draw from p_j with the same uniform
    use_p = true;
    for (int cc = 0; cc < nT; ++cc) {
      const double m = tile_mass_p<DT>(P, trow, cc, sr.m_t, sr.s_t, sm);
      if (tid == 0) sm.tot[cc] = m;
    }
    __syncthreads();
  }
  const int cstar = sm.bc[2] >= 0 ? sm.bc[2] : nT - 1;
  const double prefix = sm.dbc[0], tau = sm.dbc[1];
  __syncthreads();
  const int token = tile_draw<DT>(P, trow, drow, cstar, resid && !use_p, sr.m_t, sr.s_t, sr.m_d, sr.s_d, prefix,
                                  tau, sm);
  if (tid == 0) {
    P.out_tokens[(int64_t)b * K1 + j] = token;
    st_dev(P.darrive + b, 0);
    SeqRec z;
    memset(&z, 0, sizeof z);
    P.srec[b] = z;
  }
  for (int cc = tid; cc < nT; cc += TPB) st_dev(P.rsum + (int64_t)b * nT + cc, 0.0);
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t fault, garrive, sarrive, darrive, recs, grec, srec, cand, rsum, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int tile_of(int dtype) { return dtype == SV_BF16 ? Fmt<SV_BF16>::TILE : Fmt<SV_F32>::TILE; }

Layout layout_for(int B, int k, int V, int dtype) {
  const size_t groups = (size_t)B * (k + 1);
  const size_t nT = ((size_t)V + tile_of(dtype) - 1) / tile_of(dtype);
  Layout L;
  size_t o = 0;
  L.fault = o;   o = align256(o + sizeof(int32_t));     // fixed header, same offset for every shape
  L.garrive = o; o = align256(o + groups * sizeof(int32_t));
  L.sarrive = o; o = align256(o + (size_t)B * sizeof(int32_t));
  L.darrive = o; o = align256(o + (size_t)B * sizeof(int32_t));
  L.recs = o;    o = align256(o + groups * nT * sizeof(TileRec));
  L.grec = o;    o = align256(o + groups * sizeof(GroupRec));
  L.srec = o;    o = align256(o + (size_t)B * sizeof(SeqRec));
  L.cand = o;    o = align256(o + groups * nT * SLOTS * sizeof(uint64_t));
  L.rsum = o;    o = align256(o + (size_t)B * nT * sizeof(double));
  L.total = o;
  return L;
}

bool shape_ok(const sv_shape_t *s) {
  return s->B >= 0 && s->k >= 0 && s->V >= 1 && (s->dtype == SV_F32 || s->dtype == SV_BF16) &&
         (int64_t)s->V <= (int64_t)MAX_TILES * tile_of(s->dtype);
}

template <int DT> hipError_t launch(const Params &P, bool greedy, hipStream_t stream) {
  const unsigned items = (unsigned)((int64_t)P.B * (P.k + 1) * P.nT);
  if (greedy) {
    hipLaunchKernelGGL((sv_stream<DT, true>), dim3(items), dim3(TPB), 0, stream, P);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((sv_stream<DT, false>), dim3(items), dim3(TPB), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sv_draw<DT>), dim3((unsigned)((int64_t)P.B * P.nT)), dim3(TPB), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

extern "C" size_t spec_verify_workspace_bytes(const sv_shape_t *s) {
  if (!s || !shape_ok(s)) return 0;
  return layout_for(s->B, s->k, s->V, s->dtype).total;
}

extern "C" const char *spec_verify_error_string(int code) {
  switch (code) {
    case SV_OK: return "success";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE:
      return "invalid shape (B<0, k<0, V<1, V above 524288 for bf16 or 262144 for fp32, row stride < V, "
             "or sizes too large)";
    case SV_ERR_TEMPERATURE: return "temperature must be finite and >= 0";
    case SV_ERR_DTYPE: return "dtype must be SV_F32 or SV_BF16";
    case SV_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than spec_verify_workspace_bytes";
    case SV_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case SV_ERR_DEVICE: return "current device is not usable";
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
  if (!shape_ok(&s)) return SV_ERR_SHAPE;
  const int64_t ts = s.target_row_stride ? s.target_row_stride : s.V;
  const int64_t ds = s.draft_row_stride ? s.draft_row_stride : s.V;
  if (ts < s.V || ds < s.V) return SV_ERR_SHAPE;
  const int tile = tile_of(s.dtype);
  const int64_t nT = ((int64_t)s.V + tile - 1) / tile;
  const int64_t items = (int64_t)s.B * (s.k + 1) * nT;
  if (items > 0x7fffffffLL || (int64_t)s.B * (s.k + 2) > 0x7fffffffLL) return SV_ERR_SHAPE;
  if (!(s.temperature >= 0.f) || s.temperature == __builtin_inff()) return SV_ERR_TEMPERATURE;
  const bool greedy = s.temperature == 0.f;
  if (s.B == 0) return SV_OK;
  if (!target_logits || !accepted_len || !out_tokens || !topk_val || !topk_idx) return SV_ERR_NULL;
  if (s.k > 0 && !draft_tokens) return SV_ERR_NULL;
  if (!greedy && ((s.k > 0 && !draft_logits) || !uniforms)) return SV_ERR_NULL;
  const Layout L = layout_for(s.B, s.k, s.V, s.dtype);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;

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
  P.fault = (int32_t *)(ws + L.fault);
  P.garrive = (int32_t *)(ws + L.garrive);
  P.sarrive = (int32_t *)(ws + L.sarrive);
  P.darrive = (int32_t *)(ws + L.darrive);
  P.recs = (TileRec *)(ws + L.recs);
  P.grec = (GroupRec *)(ws + L.grec);
  P.srec = (SeqRec *)(ws + L.srec);
  P.cand = (uint64_t *)(ws + L.cand);
  P.rsum = (double *)(ws + L.rsum);
  P.B = s.B;
  P.k = s.k;
  P.V = s.V;
  P.nT = (int32_t)nT;
  P.T = greedy ? 0.f : s.temperature;
  P.scd = greedy ? 0.0 : 1.4426950408889634 / (double)s.temperature;
  P.sc = (float)P.scd;
  P.t_vec = (((uintptr_t)target_logits & 15) == 0 && ((ts * esz) & 15) == 0) ? 1 : 0;
  P.d_vec = (!greedy && s.k > 0 && ((uintptr_t)draft_logits & 15) == 0 && ((ds * esz) & 15) == 0) ? 1 : 0;

  const hipError_t e = s.dtype == SV_BF16 ? launch<SV_BF16>(P, greedy, (hipStream_t)stream)
                                          : launch<SV_F32>(P, greedy, (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}
