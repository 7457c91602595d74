// spec_verify.hip -- speculative-sampling verification for gfx950 (MI355X).
//
// One persistent, cooperatively launched kernel runs the whole step.  The
// vocabulary of every row is cut into fixed tiles (4096 entries for bf16, 2048
// for fp32: 8 KB per row either way).  A work item is one tile of one "group":
// for i < k the group is the pair (target row i, draft row i) of a sequence,
// group k is target row k alone, and in greedy mode every group is one target
// row.  Workgroups take items round-robin (item = blockIdx.x + r * gridDim.x);
// the items of a group are consecutive, so a group is spread over distinct,
// co-resident workgroups.  While a workgroup works on one item, the tiles of
// its next item are already streaming into registers.
//
// Per item:
//  A  stage the tile(s) in LDS (each thread keeps its own 16-byte vectors);
//     per-thread max and sum of exp2((x - max) * log2(e)/T) (fp32 exp and
//     per-thread fp32 sums, fp64 above the thread); reduce to a tile record and
//     publish it.
//  -- group barrier: wait until every tile of the group has published.
//  B  combine the tile records in tile order (fp64) into the row max and
//     normaliser, identical in every workgroup of the group; take the row's
//     acceptance decision; write the tile's top-32 candidates (elements at or
//     above the 32nd largest wave maximum of the row: at least 32 elements lie
//     there) to the tile's slots.  If the row is the sequence's first rejection
//     (or the bonus row after k acceptances), publish the tile's share of the
//     residual mass max(0, p - q) (or of p).
//  C  the last workgroup of the group merges the candidates into the top-32
//     (value desc, index asc); the last group of the sequence assembles it: an
//     inverse-CDF draw over the drawing row's tile masses in tile order, then
//     the crossing tile re-read and scanned element by element.
//
// Cross-workgroup data moves through the workspace with device-scope
// write-through stores and device-scope loads, ordered by waiting for the
// stores to complete before the counter that announces them is bumped.  No
// L2 write-back or invalidate is needed anywhere.
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
constexpr int NSEG = 2;                // 16-byte vectors per thread per row
constexpr int SLOTS = 32;              // top-32 candidate slots per tile
constexpr int MERGE_CAP = 512;         // candidates a group merge ranks in LDS
constexpr int TOPK = SV_TOPK;
constexpr int MAX_TILES = 128;
constexpr uint32_t SPIN_LIMIT = 1u << 19;      // about half a second of polling
constexpr float NEG_INF = -__builtin_inff();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Fmt;
template <> struct Fmt<SV_BF16> { static constexpr int E = 2, W = 8, TILE = TPB * NSEG * 8; };
template <> struct Fmt<SV_F32> { static constexpr int E = 4, W = 4, TILE = TPB * NSEG * 4; };

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
  int32_t argmax;          // top-1 index of the target row (written by the merge)
  int32_t pad;
};

// arrive2 counts arrivals in its high half and candidate overflows in its low
// half; dec: 0 pending, 1 drafted token accepted, 2 rejected or data error
struct GroupSync { int32_t arrive1, arrive2, dec, pad; };

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
  uint64_t *cand;                      // [group][tile][SLOTS] candidate keys, 0 = empty
  int32_t B, k, V, nT, items;
  float T, sc;                         // sc = log2(e) / T
  double scd;
  int32_t t_vec, d_vec;                // rows 16-byte aligned
};

struct Smem {
  union {
    u32x4 tile[2][NSEG][TPB];          // staged tile: [target, draft][vector][thread]
    uint64_t keys[MERGE_CAP];          // group merge: candidate keys
    struct {                           // exact top-32 fallback
      uint32_t hist[2048];
      int32_t part[TPB];
      uint64_t list[TOPK];
    } fb;
  };
  union {
    uint32_t wkeys[NWAVE * MAX_TILES]; // phase B: wave maxima of the row
    double tot[MAX_TILES];             // sequence assembly: tile masses
  };
  float f[4][NWAVE];
  uint32_t u[2][NWAVE];
  int32_t i[4][NWAVE];
  double d[4][NWAVE];
  int32_t bc[8];
  double dbc[4];
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
// Poll a device counter until it reaches `target`.  A wait that never ends
// would be a bug: after SPIN_LIMIT polls (or once another wait has given up)
// mark the fault word and return, so the grid always drains.
__device__ __forceinline__ void wait_at_least(const int32_t *p, int target, int32_t *fault) {
  uint32_t spins = 0;
  while (ld_dev(p) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > SPIN_LIMIT || ((spins & 255) == 0 && ld_dev(fault))) {
      atomicOr(fault, 1);
      return;
    }
  }
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

template <int DT, bool GREEDY>
__device__ __forceinline__ void fetch(const Params &P, int item, u32x4 (&nt)[NSEG], u32x4 (&nd)[NSEG]) {
  const Geo G = geo<DT, GREEDY>(P, item);
  load_tile<DT>(G.trow, G.c, P.V, P.t_vec, nt);
  if (G.pair) load_tile<DT>(G.drow, G.c, P.V, P.d_vec, nd);
}

// Each thread stages its own vectors and only ever reads those back, so no
// barrier is needed between staging and use.
__device__ __forceinline__ void stage(Smem &sm, const u32x4 (&t)[NSEG], const u32x4 (&d)[NSEG], bool pair) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    sm.tile[0][s][threadIdx.x] = t[s];
    if (pair) sm.tile[1][s][threadIdx.x] = d[s];
  }
}

template <int DT> __device__ __forceinline__ float thread_max(const Smem &sm, int r) {
  float m = NEG_INF;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const u32x4 v = sm.tile[r][s][threadIdx.x];
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) m = fmaxf(m, unpack<DT>(v, w));
  }
  return m;
}

template <int DT> __device__ __forceinline__ bool thread_has_nan(const Smem &sm, int r) {
  bool nan = false;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const u32x4 v = sm.tile[r][s][threadIdx.x];
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) { const float x = unpack<DT>(v, w); nan |= !(x == x); }
  }
  return nan;
}

// exp2((x - m) * sc) of one element; a thread whose slice is all -inf uses 0 as m
__device__ __forceinline__ float scaled_exp(float x, float m, float sc) {
  const float ms = (m == NEG_INF) ? 0.f : m;
  return __builtin_amdgcn_exp2f((x - ms) * sc);
}

// Sequential fp32 sum of the thread's scaled exps; flags NaN / +inf.
template <int DT>
__device__ __forceinline__ float thread_expsum(const Smem &sm, int r, float m, float sc, int &flags) {
  float s = 0.f;
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    const u32x4 v = sm.tile[r][g][threadIdx.x];
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) s += scaled_exp(unpack<DT>(v, w), m, sc);
  }
  flags = 0;
  if (!(s == s)) flags = thread_has_nan<DT>(sm, r) ? SV_STATUS_NAN : SV_STATUS_POSINF;
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

// Sequential fp32 mass of each of the thread's vectors of the staged tile.
template <int DT>
__device__ __forceinline__ void seg_masses(const Smem &sm, bool resid, float mt, float md, float at, float ad,
                                           float sc, float (&seg)[NSEG]) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const u32x4 vt = sm.tile[0][s][threadIdx.x];
    const u32x4 vd = resid ? sm.tile[1][s][threadIdx.x] : vt;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) a += elem_mass<DT>(vt, vd, w, resid, mt, md, at, ad, sc);
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

// Top-32 of a target row by exact radix selection over the whole row (used
// when the candidate slots overflowed).  Rank 0's index goes to sm.bc[7].
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
    if (rank == 0) sm.bc[7] = cand_index(ka);
  }
  for (int r = need + tid; r < TOPK; r += TPB) { oidx[r] = -1; oval[r] = NEG_INF; }
  __syncthreads();
}

// Top-32 of a target row from the candidate slots of its tiles (the last
// workgroup of the group runs it).  Every slot read non-empty is cleared.
template <int DT>
__device__ void merge_top32(const Params &P, int g, int row, bool overflow, bool nanrow, const char *trow,
                            Smem &sm) {
  const int tid = threadIdx.x;
  float *oval = P.topk_val + (int64_t)row * TOPK;
  int32_t *oidx = P.topk_idx + (int64_t)row * TOPK;
  if (tid == 0) { sm.bc[6] = 0; sm.bc[7] = -1; }
  __syncthreads();
  uint64_t *slots = P.cand + (int64_t)g * P.nT * SLOTS;
  for (int a = tid; a < P.nT * SLOTS; a += TPB) {
    const uint64_t key = ld_dev(slots + a);
    if (key) {
      st_dev(slots + a, (uint64_t)0);
      const int pos = atomicAdd(&sm.bc[6], 1);
      if (pos < MERGE_CAP) sm.keys[pos] = key;
    }
  }
  __syncthreads();
  const int n = sm.bc[6];
  if (nanrow) {
    for (int r = tid; r < TOPK; r += TPB) { oval[r] = __builtin_nanf(""); oidx[r] = -1; }
  } else if (overflow || n > MERGE_CAP) {
    topk_exact<DT>(trow, P.V, oval, oidx, sm);
  } else {
    for (int a = tid; a < n; a += TPB) {
      const uint64_t ka = sm.keys[a];
      int rank = 0;
      for (int jj = 0; jj < n; ++jj) rank += sm.keys[jj] > ka;
      if (rank < TOPK) {
        oidx[rank] = cand_index(ka);
        oval[rank] = cand_value(ka);
        if (rank == 0) sm.bc[7] = cand_index(ka);
      }
    }
    for (int r = n + tid; r < TOPK; r += TPB) { oval[r] = NEG_INF; oidx[r] = -1; }
  }
  __syncthreads();
}

// Stage tile c of a row (and of the draft row when resid) and compute the
// per-thread scales; same arithmetic as the row's own items used.
template <int DT>
__device__ __forceinline__ void stage_row_tile(const Params &P, const char *trow, const char *drow, int c, bool resid,
                                               float m_t, double s_t, float m_d, double s_d, Smem &sm, float &mt,
                                               float &md, float &at, float &ad) {
  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(trow, c, P.V, P.t_vec, rt);
  if (resid) load_tile<DT>(drow, c, P.V, P.d_vec, rd);
  __syncthreads();               // the staging area may still hold another use's data
  stage(sm, rt, rd, resid);
  mt = thread_max<DT>(sm, 0);
  md = resid ? thread_max<DT>(sm, 1) : NEG_INF;
  at = prob_scale(mt, m_t, s_t, P.sc);
  ad = resid ? prob_scale(md, m_d, s_d, P.sc) : 0.f;
}

// Draw by inverse CDF inside one tile: the first element (ascending index) of
// positive mass whose cumulative mass prefix + (scan base + running fp32 sum)
// exceeds tau; if rounding leaves none, the tile's last positive-mass element.
template <int DT>
__device__ int tile_draw(const Params &P, const char *trow, const char *drow, int c, bool resid, float m_t,
                         double s_t, float m_d, double s_d, double prefix, double tau, Smem &sm) {
  constexpr int W = Fmt<DT>::W;
  float mt, md, at, ad;
  stage_row_tile<DT>(P, trow, drow, c, resid, m_t, s_t, m_d, s_d, sm, mt, md, at, ad);
  float seg[NSEG];
  seg_masses<DT>(sm, resid, mt, md, at, ad, P.sc, seg);
  double base[NSEG];
  tile_scan(seg, base, sm);
  int first = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const u32x4 vt = sm.tile[0][s][threadIdx.x];
    const u32x4 vd = resid ? sm.tile[1][s][threadIdx.x] : vt;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mval = elem_mass<DT>(vt, vd, w, resid, mt, md, at, ad, P.sc);
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

// Target mass p of one tile (same arithmetic as tile_draw without a draft row).
template <int DT>
__device__ double tile_mass_p(const Params &P, const char *trow, int c, float m_t, double s_t, Smem &sm) {
  float mt, md, at, ad;
  stage_row_tile<DT>(P, trow, nullptr, c, false, m_t, s_t, 0.f, 1.0, sm, mt, md, at, ad);
  float seg[NSEG];
  seg_masses<DT>(sm, false, mt, md, at, ad, P.sc, seg);
  double base[NSEG];
  return tile_scan(seg, base, sm);
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

// Sampling-mode sequence assembly (run by the last group of the sequence).
template <int DT>
__device__ void finish_sampling(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1, nT = P.nT;
  int st = 0, j = k;
  for (int i = tid; i <= k; i += TPB) {
    const GroupRec r = ld_rec(P.grec + (int64_t)b * K1 + i);
    st |= r.flags;
    if (i < k && !r.accept && i < j) j = i;
  }
  for (int i = tid; i < k + 2; i += TPB) {
    const float u = P.uniforms[(int64_t)b * (k + 2) + i];
    if (!(u >= 0.f && u < 1.f)) st |= SV_STATUS_BAD_UNIFORM;
  }
  if (tid == 0 && ld_dev(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
  block_or_min(st, j, sm);
  int token = -1;
  if (!st) {
    const int g = b * K1 + j;
    const bool resid = j < k;
    const GroupRec gr = ld_rec(P.grec + g);
    for (int c = tid; c < nT; c += TPB) sm.tot[c] = ld_dev(P.rsum + (int64_t)g * nT + c);
    __syncthreads();
    const double u = (double)P.uniforms[(int64_t)b * (k + 2) + (resid ? k : k + 1)];
    const char *trow = P.target + ((int64_t)b * K1 + j) * P.tstride * Fmt<DT>::E;
    const char *drow = resid ? P.draft + ((int64_t)b * k + j) * P.dstride * Fmt<DT>::E : nullptr;
    bool use_p = false;
    for (int attempt = 0; attempt < 2; ++attempt) {
      if (tid == 0) {
        double R = 0.0;
        for (int c = 0; c < nT; ++c) R += sm.tot[c];
        const double tau = u * R;
        double Pc = 0.0;
        int cs = -1;
        for (int c = 0; c < nT; ++c) {
          const double nx = Pc + sm.tot[c];
          if (nx > tau) { cs = c; break; }
          Pc = nx;
        }
        sm.bc[2] = cs;
        sm.dbc[0] = Pc;
        sm.dbc[1] = tau;
      }
      __syncthreads();
      if (sm.bc[2] >= 0 || attempt == 1) break;
      // no residual mass left (rounding): draw from p_j with the same uniform
      use_p = true;
      for (int c = 0; c < nT; ++c) {
        const double m = tile_mass_p<DT>(P, trow, c, gr.m_t, gr.s_t, sm);
        if (tid == 0) sm.tot[c] = m;
      }
      __syncthreads();
    }
    const int cstar = sm.bc[2] >= 0 ? sm.bc[2] : nT - 1;
    const double prefix = sm.dbc[0], tau = sm.dbc[1];
    __syncthreads();
    token = tile_draw<DT>(P, trow, drow, cstar, resid && !use_p, gr.m_t, gr.s_t, gr.m_d, gr.s_d, prefix, tau, sm);
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

// Greedy-mode sequence assembly: argmax-prefix match on the rows' top-1 entries.
__device__ void finish_greedy(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1;
  int st = 0, j = k;
  for (int i = tid; i <= k; i += TPB) {
    const int64_t g = (int64_t)b * K1 + i;
    st |= ld_dev(&P.grec[g].flags);
    if (i < k) {
      const int32_t x = P.tokens[(int64_t)b * k + i];
      if (x < 0 || x >= P.V) st |= SV_STATUS_BAD_TOKEN;
      else if (x != ld_dev(&P.grec[g].argmax) && i < j) j = i;
    }
  }
  if (tid == 0 && ld_dev(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
  block_or_min(st, j, sm);
  const int aj = st ? -1 : ld_dev(&P.grec[(int64_t)b * K1 + j].argmax);
  if (tid == 0) {
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
  }
  for (int i = tid; i < K1; i += TPB) {
    int v = -1;
    if (!st) v = i < j ? P.tokens[(int64_t)b * k + i] : (i == j ? aj : -1);
    P.out_tokens[(int64_t)b * K1 + i] = v;
  }
}

// Sequence arrival of a group; the last group of the sequence assembles it and
// clears the sequence's records.
template <int DT, bool GREEDY>
__device__ void sequence_arrival(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int K1 = P.k + 1, nT = P.nT;
  stores_done();
  __syncthreads();
  if (tid == 0) sm.bc[5] = add_dev(P.seqctr + b, 1);
  __syncthreads();
  if (sm.bc[5] != K1 - 1) return;
  if (GREEDY) finish_greedy(P, b, sm);
  else finish_sampling<DT>(P, b, sm);
  __syncthreads();
  zero_recs(P.grec + (int64_t)b * K1, K1);
  if (!GREEDY)
    for (int a = tid; a < K1 * nT; a += TPB) st_dev(P.rsum + (int64_t)b * K1 * nT + a, 0.0);
  for (int a = tid; a < K1; a += TPB) st_dev(&P.sync[(int64_t)b * K1 + a].dec, 0);
  if (tid == 0) st_dev(P.seqctr + b, 0);
  __syncthreads();
}

template <int DT, bool GREEDY>
__device__ __forceinline__ void process_item(const Params &P, int item, u32x4 (&nt)[NSEG], u32x4 (&nd)[NSEG],
                                             Smem &sm) {
  constexpr int W = Fmt<DT>::W, TILE = Fmt<DT>::TILE;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1, V = P.V;
  const Geo G = geo<DT, GREEDY>(P, item);
  const int g = G.g, c = G.c, b = G.b, i = G.i;
  const bool pair = G.pair;

  // drafted token and its two logits: every workgroup of the group decides
  int32_t x = -1;
  float tx = 0.f, dx = 0.f;
  if (pair && tid == 0) {
    x = P.tokens[(int64_t)b * k + i];
    if (x >= 0 && x < V) { tx = load_elem<DT>(G.trow, x); dx = load_elem<DT>(G.drow, x); }
  }
  stage(sm, nt, nd, pair);

  // ---------------- phase A: per-thread and per-tile statistics
  const float mt = thread_max<DT>(sm, 0);
  const float md = pair ? thread_max<DT>(sm, 1) : NEG_INF;
  int ft = 0, fd = 0;
  float st = 0.f, sd = 0.f;
  if (!GREEDY) {
    st = thread_expsum<DT>(sm, 0, mt, P.sc, ft);
    if (pair) sd = thread_expsum<DT>(sm, 1, md, P.sc, fd);
  } else {
    ft = thread_has_nan<DT>(sm, 0) ? SV_STATUS_NAN : 0;
  }
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

  // ---------------- publish the tile record; start the next item's loads;
  // wait for the whole group
  if (tid == 0) {
    TileRec r;
    r.m_t = m_ct; r.m_d = m_cd; r.s_t = s_ct; r.s_d = s_cd;
    for (int w = 0; w < NWAVE; ++w) r.wkey[w] = sm.u[0][w];
    r.flags_t = f_ct; r.flags_d = f_cd;
    st_rec(P.recs + item, r);
    stores_done();
    const int old1 = add_dev(&P.sync[g].arrive1, 1);
    if (old1 < 0 || old1 >= nT) atomicOr(P.fault, 2);      // workspace was not zero-filled
  }
  if (item + (int)gridDim.x < P.items) fetch<DT, GREEDY>(P, item + gridDim.x, nt, nd);
  if (tid == 0) wait_at_least(&P.sync[g].arrive1, nT, P.fault);
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  // ---------------- phase B: row statistics, identical in every workgroup
  // nT <= TPB: thread cc holds the record of tile cc
  TileRec rec;
  const bool own = tid < nT;
  if (own) {
    rec = ld_rec(P.recs + (int64_t)g * nT + tid);
    for (int w = 0; w < NWAVE; ++w) sm.wkeys[tid * NWAVE + w] = rec.wkey[w];
  } else {
    rec.m_t = NEG_INF; rec.m_d = NEG_INF; rec.s_t = 0.0; rec.s_d = 0.0; rec.flags_t = 0; rec.flags_d = 0;
  }
  {
    const float a = wave_max(rec.m_t), d = wave_max(rec.m_d);
    const int fa = wave_or(rec.flags_t), fb = wave_or(rec.flags_d);
    if (lane == 0) { sm.f[2][wid] = a; sm.f[3][wid] = d; sm.i[2][wid] = fa; sm.i[3][wid] = fb; }
  }
  __syncthreads();
  float m_rt = sm.f[2][0], m_rd = sm.f[3][0];
  int f_rt = sm.i[2][0], f_rd = sm.i[3][0];
  for (int w = 1; w < NWAVE; ++w) {
    m_rt = fmaxf(m_rt, sm.f[2][w]); m_rd = fmaxf(m_rd, sm.f[3][w]);
    f_rt |= sm.i[2][w]; f_rd |= sm.i[3][w];
  }
  if (!GREEDY) {
    double a = 0.0, d = 0.0;
    if (own && rec.m_t != NEG_INF) a = rec.s_t * (double)__builtin_amdgcn_exp2f((rec.m_t - m_rt) * P.sc);
    if (own && pair && rec.m_d != NEG_INF) d = rec.s_d * (double)__builtin_amdgcn_exp2f((rec.m_d - m_rd) * P.sc);
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
  double s_rt = 0.0, s_rd = 0.0;
  if (!GREEDY) for (int w = 0; w < NWAVE; ++w) { s_rt += sm.d[2][w]; s_rd += sm.d[3][w]; }
  const uint32_t L = sm.u[1][0];
  // one data-error bit per row: NaN before +inf before an empty row
  f_rt = (f_rt & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rt;
  f_rd = (f_rd & SV_STATUS_NAN) ? SV_STATUS_NAN : f_rd;
  if (!GREEDY && m_rt == NEG_INF && !f_rt) f_rt = SV_STATUS_EMPTY_ROW;
  if (pair && m_rd == NEG_INF && !f_rd) f_rd = SV_STATUS_EMPTY_ROW;

  // acceptance decision of the row (one thread; tile 0 publishes it)
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
    sm.bc[0] = fl;
    sm.bc[1] = acc;
    if (c == 0) {
      GroupRec gr;
      gr.s_t = s_rt; gr.s_d = s_rd; gr.m_t = m_rt; gr.m_d = m_rd;
      gr.flags = fl; gr.accept = acc; gr.argmax = -1; gr.pad = 0;
      st_rec(P.grec + g, gr);
      if (!GREEDY) {
        st_dev(&P.sync[g].dec, (fl || !acc) ? 2 : 1);
        if (P.lse_t) P.lse_t[(int64_t)b * K1 + i] = (float)((double)m_rt / (double)P.T + log(s_rt));
        if (pair) {
          if (P.p_tok) P.p_tok[(int64_t)b * k + i] = pt;
          if (P.q_tok) P.q_tok[(int64_t)b * k + i] = qt;
          if (P.lse_d) P.lse_d[(int64_t)b * k + i] = (float)((double)m_rd / (double)P.T + log(s_rd));
        }
      }
    }
  }

  // top-32 candidates of the target row: elements at or above the bound go to
  // this tile's slots in element order
  {
    const float Lf = key_value(L);
    const int lim = V - c * TILE;                        // tile positions < lim exist
    uint32_t mask = 0;
    if (has_elem && (L == 0u || mt >= Lf)) {
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        const u32x4 v = sm.tile[0][s][tid];
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float xv = unpack<DT>(v, w);
          if (tpos<DT>(s, w) < lim && (L == 0u || xv >= Lf)) mask |= 1u << (s * W + w);
        }
      }
    }
    const int cnt = __popc(mask);
    const int inc = wave_incl_int(cnt, lane);
    if (lane == 63) sm.i[0][wid] = inc;
    __syncthreads();
    int slot = inc - cnt, total = 0;
    for (int w = 0; w < NWAVE; ++w) { if (w < wid) slot += sm.i[0][w]; total += sm.i[0][w]; }
    uint64_t *dst = P.cand + ((int64_t)g * nT + c) * SLOTS;
    while (mask) {
      const int bit = __builtin_ctz(mask);
      mask &= mask - 1;
      const int s = bit / W, w = bit - s * W;
      const float xv = unpack<DT>(sm.tile[0][s][tid], w);
      if (slot < SLOTS) st_dev(dst + slot, cand_key(xv, c * TILE + tpos<DT>(s, w)));
      ++slot;
    }
    if (tid == 0) sm.bc[3] = total > SLOTS ? 1 : 0;
  }
  __syncthreads();
  const int overflow = sm.bc[3];

  // the row whose token is drawn (first rejection, or the bonus row after k
  // acceptances) publishes its tiles' masses for the inverse-CDF draw
  if (!GREEDY) {
    if (tid == 0) {
      int need = 0;
      if (!sm.bc[0] && !(pair && sm.bc[1])) {
        need = 1;
        for (int l = 0; l < i; ++l) {
          const int32_t *dp = &P.sync[(int64_t)b * K1 + l].dec;
          wait_at_least(dp, 1, P.fault);
          if (ld_dev(dp) != 1) { need = 0; break; }
        }
      }
      sm.bc[2] = need;
    }
    __syncthreads();
    if (sm.bc[2]) {
      const float at = prob_scale(mt, m_rt, s_rt, P.sc);
      const float ad = pair ? prob_scale(md, m_rd, s_rd, P.sc) : 0.f;
      float seg[NSEG];
      seg_masses<DT>(sm, pair, mt, md, at, ad, P.sc, seg);
      double base[NSEG];
      const double tot = tile_scan(seg, base, sm);
      if (tid == 0) st_dev(P.rsum + item, tot);
    }
  }

  // ---------------- group arrival; the last workgroup finishes the group
  stores_done();
  __syncthreads();
  if (tid == 0) {
    const int old = add_dev(&P.sync[g].arrive2, (1 << 16) | overflow);
    sm.bc[4] = ((old >> 16) == nT - 1) ? 1 + ((old & 0xffff) + overflow > 0 ? 1 : 0) : 0;
  }
  __syncthreads();
  const int last = sm.bc[4];
  if (!last) return;
  const bool any_overflow = last == 2;

  if (!GREEDY) sequence_arrival<DT, GREEDY>(P, b, sm);
  merge_top32<DT>(P, g, b * K1 + i, any_overflow, (f_rt & SV_STATUS_NAN) != 0, G.trow, sm);
  if (GREEDY && tid == 0) st_dev(&P.grec[g].argmax, sm.bc[7]);
  // every workgroup of the group is past both barriers: clear the group's
  // records and counters so the call leaves the workspace zero-filled
  zero_recs(P.recs + (int64_t)g * nT, nT);
  if (tid == 0) {
    st_dev(&P.sync[g].arrive1, 0);
    st_dev(&P.sync[g].arrive2, 0);
  }
  if (GREEDY) sequence_arrival<DT, GREEDY>(P, b, sm);
}

template <int DT, bool GREEDY>
__global__ __launch_bounds__(TPB) void spec_verify_kernel(Params P) {
  __shared__ Smem sm;
  int item = blockIdx.x;
  if (item >= P.items) return;
  u32x4 nt[NSEG], nd[NSEG];            // the tiles of the item about to be processed
  fetch<DT, GREEDY>(P, item, nt, nd);
  for (; item < P.items; item += gridDim.x) {
    process_item<DT, GREEDY>(P, item, nt, nd, sm);
    stores_done();
    __syncthreads();
  }
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t fault, sync, seqctr, recs, rsum, grec, cand, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int tile_of(int dtype) { return dtype == SV_BF16 ? Fmt<SV_BF16>::TILE : Fmt<SV_F32>::TILE; }

Layout layout_for(int B, int k, int V, int dtype) {
  const size_t groups = (size_t)B * (k + 1);
  const size_t nT = ((size_t)V + tile_of(dtype) - 1) / tile_of(dtype);
  Layout L;
  size_t o = 0;
  L.fault = o;  o = align256(o + sizeof(int32_t));      // fixed header, same offset for every shape
  L.sync = o;   o = align256(o + groups * sizeof(GroupSync));
  L.seqctr = o; o = align256(o + (size_t)B * sizeof(int32_t));
  L.recs = o;   o = align256(o + groups * nT * sizeof(TileRec));
  L.rsum = o;   o = align256(o + groups * nT * sizeof(double));
  L.grec = o;   o = align256(o + groups * sizeof(GroupRec));
  L.cand = o;   o = align256(o + groups * nT * SLOTS * sizeof(uint64_t));
  L.total = o;
  return L;
}

bool shape_ok(const sv_shape_t *s) {
  return s->B >= 0 && s->k >= 0 && s->V >= 1 && (s->dtype == SV_F32 || s->dtype == SV_BF16) &&
         (int64_t)s->V <= (int64_t)MAX_TILES * tile_of(s->dtype);
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
  P.T = greedy ? 0.f : s.temperature;
  P.scd = greedy ? 0.0 : 1.4426950408889634 / (double)s.temperature;
  P.sc = (float)P.scd;
  P.t_vec = (((uintptr_t)target_logits & 15) == 0 && ((ts * esz) & 15) == 0) ? 1 : 0;
  P.d_vec = (!greedy && s.k > 0 && ((uintptr_t)draft_logits & 15) == 0 && ((ds * esz) & 15) == 0) ? 1 : 0;

  const int variant = (s.dtype == SV_BF16 ? 2 : 0) + (greedy ? 1 : 0);
  const int64_t resident = (int64_t)dev->occ[variant] * dev->cus;
  int64_t grid = resident;
  if (const char *lim = getenv("SV_GRID_LIMIT")) {
    const long v = strtol(lim, nullptr, 10);
    if (v > 0 && v < grid) grid = v;
  }
  if (grid < nT) grid = nT;                      // a group must fit on the device at once
  if (grid > resident) return SV_ERR_DEVICE;
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
