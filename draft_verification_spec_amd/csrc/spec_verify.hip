// spec_verify.hip -- speculative-sampling verification for gfx950 (MI355X).
//
// Two plain launches; no workgroup ever waits for another.
//
//  sv_stream  one workgroup per (group, tile).  A group is, for i < k, the pair
//             (target row i, draft row i) of a sequence and, for i == k, target
//             row k alone; in greedy mode every group is one target row.  Tiles
//             are fixed vocabulary slices (4096 bf16 or 2048 fp32 entries, 8 KB
//             of each row).  Each workgroup streams its tile(s) once with 128-bit
//             loads and publishes a tile record:
//               - max and sum of exp2((x - max) * log2(e)/T) of each row part
//                 (fp32 exp, per-thread fp32 sums, fp64 above the thread);
//               - the tile's 8 largest lane maxima (a lane owns 16 elements of
//                 a bf16 tile, 8 of an fp32 tile);
//             and, as top-32 candidates, the elements at or above the 8th of
//             those lane maxima.
//             The last workgroup of a group to publish combines the records in
//             tile order, takes the acceptance decision and merges the top-32.
//             The 32nd largest of all the tiles' lane maxima is a lower bound of
//             the row's 32nd largest element (32 distinct elements reach it).
//             Candidates at or above it are ranked; a tile whose 8th lane
//             maximum lies above the bound may hold further elements above it
//             and is rescanned, as is a tile whose candidates overflowed.
//             The last group of a sequence finds the first rejection j (greedy:
//             the first draft that differs from the argmax).
//  sv_draw    sampling only.  After a rejection at j every tile of pair row j
//             publishes its residual mass max(0, p - q); the last one draws by
//             inverse CDF over the tile masses in tile order and rescans the
//             crossing tile.  After k acceptances a single workgroup draws from
//             p_k, whose tile masses the merge of row k has already published.
//
// Wave-level reductions and scans run on DPP row shifts and broadcasts in a
// fixed order, so every reduction is deterministic.  Cross-workgroup data within
// a launch moves through the workspace with device-scope write-through stores
// and device-scope loads, ordered by waiting for the stores to complete before
// the counter that announces them is bumped.  No workgroup waits for another,
// so any dispatch order and any occupancy are safe.
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
constexpr int LIST = 8;                // lane maxima a tile record keeps
constexpr int SLOTS = 16;              // candidate slots per tile
constexpr int MERGE_CAP = 512;         // candidates a row merge ranks in LDS
constexpr int TOPK = SV_TOPK;
constexpr int MAX_TILES = 128;
constexpr int KEYS_PT = MAX_TILES * SLOTS / TPB;   // candidate slots per merge thread
constexpr int RECW_PT = MAX_TILES * 8 / TPB;       // tile-record words per merge thread
constexpr int TOPS_PL = MAX_TILES * LIST / 64;     // lane maxima per lane in the bound search
constexpr float NEG_INF = -__builtin_inff();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E: bytes per element; W: elements per 16-byte vector; TILE: elements per
// tile; LOW / BITS: ordered keys of this format leave LOW in their low bits,
// and only the top BITS bits separate values.
template <int DT> struct Fmt;
template <> struct Fmt<SV_BF16> {
  static constexpr int E = 2, W = 8, TILE = TPB * NSEG * 8, BITS = 16;
  static constexpr uint32_t LOW = 0xffffu;
};
template <> struct Fmt<SV_F32> {
  static constexpr int E = 4, W = 4, TILE = TPB * NSEG * 4, BITS = 32;
  static constexpr uint32_t LOW = 0u;
};

// Published per (group, tile) by sv_stream.
struct TileRec {
  float m_t, m_d;          // tile max of the target / draft row part
  double s_t, s_d;         // sum exp2((x - m) * sc) over the tile part
  int32_t flags_t, flags_d;
  uint32_t top[LIST];      // ordered keys of the tile's largest lane maxima, descending (0: no lane)
};
static_assert(sizeof(TileRec) == 64, "tile record");

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
  int32_t *ovf;                        // [group][tile] 1: more candidates than SLOTS
  double *rsum;                        // [sequence][tile] residual masses of the drawing row
  double *psum;                        // [sequence][tile] target masses of row k
  int32_t B, k, V, nT;
  float T, sc;                         // sc = log2(e) / T
  double scd;
  int32_t t_vec, d_vec;                // rows 16-byte aligned
};

struct Smem {
  union {
    uint32_t w8[NWAVE * LIST];         // stream: each wave's largest lane maxima
    struct {
      TileRec rec[MAX_TILES];          // row merge: the group's tile records
      uint64_t keys[MERGE_CAP];        // row merge: candidates at or above the bound
    } m;
    struct {                           // exact top-32 fallback
      uint32_t hist[2048];
      int32_t part[TPB];
      uint64_t list[TOPK];
    } fb;
    double tot[MAX_TILES];             // draw: tile masses
  };
  float f[4][NWAVE];
  int32_t i[4][NWAVE];
  double d[4][NWAVE];
  int32_t bc[8];
  double dbc[8];
  uint64_t rescan[2];                  // row merge: tiles to rescan
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

// ---- wave primitives on DPP.  A lane whose DPP source is outside its row, or
// that the row / bank mask leaves out, receives the identity `old`.
template <int CTRL, int RM, int BM> __device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, RM, BM, false);
}
template <int CTRL, int RM, int BM> __device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp<CTRL, RM, BM>(0u, (uint32_t)u);
  const uint32_t hi = dpp<CTRL, RM, BM>(0u, (uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, ((uint64_t)readlane((uint32_t)(u >> 32), l) << 32) | readlane((uint32_t)u, l));
}
// Reduction over the wave, returned to every lane: neighbours, then groups of
// 4 and 8 and whole rows of 16, then the four rows (lane 63 ends with all).
template <class Op> __device__ __forceinline__ uint32_t wave_red(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp<0x111, 0xf, 0xf>(id, v));   // row_shr:1
  v = op(v, dpp<0x112, 0xf, 0xf>(id, v));   // row_shr:2
  v = op(v, dpp<0x114, 0xf, 0xe>(id, v));   // row_shr:4, banks 1-3
  v = op(v, dpp<0x118, 0xf, 0xc>(id, v));   // row_shr:8, banks 2-3
  v = op(v, dpp<0x142, 0xa, 0xf>(id, v));   // row_bcast:15 into rows 1, 3
  v = op(v, dpp<0x143, 0xc, 0xf>(id, v));   // row_bcast:31 into rows 2, 3
  return readlane(v, 63);
}
struct OpMaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct OpMaxI { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return (int)a > (int)b ? a : b; } };
struct OpMinI { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return (int)a < (int)b ? a : b; } };
struct OpOr { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
struct OpMaxF {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }
};
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) { return wave_red(v, 0u, OpMaxU()); }
__device__ __forceinline__ int wave_max_i(int v) { return (int)wave_red((uint32_t)v, 0x80000000u, OpMaxI()); }
__device__ __forceinline__ int wave_min_i(int v) { return (int)wave_red((uint32_t)v, 0x7fffffffu, OpMinI()); }
__device__ __forceinline__ int wave_or(int v) { return (int)wave_red((uint32_t)v, 0u, OpOr()); }
__device__ __forceinline__ float wave_max_f(float v) {
  return __uint_as_float(wave_red(__float_as_uint(v), 0xff800000u, OpMaxF()));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0x111, 0xf, 0xf>(v);
  v += dpp_d<0x112, 0xf, 0xf>(v);
  v += dpp_d<0x114, 0xf, 0xe>(v);
  v += dpp_d<0x118, 0xf, 0xc>(v);
  v += dpp_d<0x142, 0xa, 0xf>(v);
  v += dpp_d<0x143, 0xc, 0xf>(v);
  return readlane_d(v, 63);
}
// Inclusive prefix sum over the wave's lanes: windows of 4 within a row, then
// 8 and 16, then earlier rows.
__device__ __forceinline__ double wave_scan_d(double x) {
  double v = x + dpp_d<0x111, 0xf, 0xf>(x);
  v += dpp_d<0x112, 0xf, 0xf>(x);
  v += dpp_d<0x113, 0xf, 0xf>(x);
  v += dpp_d<0x114, 0xf, 0xe>(v);
  v += dpp_d<0x118, 0xf, 0xc>(v);
  v += dpp_d<0x142, 0xa, 0xf>(v);
  v += dpp_d<0x143, 0xc, 0xf>(v);
  return v;
}
// value of the previous lane of the wave (0 in lane 0)
__device__ __forceinline__ double wave_prev_d(double v) { return dpp_d<0x138, 0xf, 0xf>(v); }

// The LIST largest keys among the wave's lanes, descending: lane r < LIST
// receives the r-th (0 where fewer lanes hold a nonzero key).  Equal keys of
// different lanes count separately.
__device__ __forceinline__ uint32_t wave_top_list(uint32_t key, int lane) {
  uint32_t mine = 0;
#pragma unroll
  for (int r = 0; r < LIST; ++r) {
    const uint32_t m = wave_max_u(key);
    const uint64_t hit = __ballot(key == m && m != 0u);
    const int sel = hit ? __builtin_ctzll(hit) : 64;
    if (lane == sel) key = 0u;
    if (lane == r) mine = m;
  }
  return mine;
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

// s * exp2((m - M) * sc) in fp64: a partial sum relative to m, rescaled to M
__device__ __forceinline__ double rescale(double s, float m, float M, float sc) {
  return m == NEG_INF ? 0.0 : s * (double)__builtin_amdgcn_exp2f((m - M) * sc);
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
  double prev[NSEG];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const double inc = wave_scan_d((double)seg[s]);
    prev[s] = wave_prev_d(inc);
    if (lane == 63) sm.d[s][wid] = inc;
  }
  __syncthreads();
  double acc = 0.0;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    double off = 0.0, tot = 0.0;
    for (int w = 0; w < NWAVE; ++w) {
      if (w < wid) off += sm.d[s][w];
      tot += sm.d[s][w];
    }
    base[s] = acc + (off + prev[s]);
    acc = acc + tot;
  }
  __syncthreads();
  return acc;
}

// Block-wide OR and MIN.
__device__ __forceinline__ void block_or_min(int &o, int &m, Smem &sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  o = wave_or(o);
  m = wave_min_i(m);
  if (lane == 0) { sm.i[2][wid] = o; sm.i[3][wid] = m; }
  __syncthreads();
  o = sm.i[2][0];
  m = sm.i[3][0];
  for (int w = 1; w < NWAVE; ++w) { o |= sm.i[2][w]; m = sm.i[3][w] < m ? sm.i[3][w] : m; }
  __syncthreads();
}

// Top-32 of a target row by exact radix selection over the whole row (used
// when more candidates reach the bound than the merge holds: heavy ties).
// Rank 0's index goes to sm.bc[6].
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

// Sequence assembly in sv_stream (run by the last group of the sequence):
// greedy emits everything; sampling emits all but the drawn token and hands
// the drawing row to sv_draw.
template <bool GREEDY>
__device__ void seq_finish(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1;
  const bool small = k + 2 <= TPB;           // one entry per thread: no reloads
  // one round of loads: group records, drafted tokens, uniforms, the fault word
  int st = 0, j = k;
  GroupRec mine = {};
  int32_t tok = 0;
  float uu = 0.5f;
  for (int i0 = 0; i0 < k + 2; i0 += TPB) {
    const int i = i0 + tid;
    GroupRec r = {};
    if (i < K1) r = ld_rec(P.grec + (int64_t)b * K1 + i);
    const int32_t x = i < k ? P.tokens[(int64_t)b * k + i] : 0;
    const float u = (!GREEDY && i < k + 2) ? P.uniforms[(int64_t)b * (k + 2) + i] : 0.5f;
    if (i < K1) {
      st |= r.flags;
      if (i < k) {
        if (GREEDY) {
          if (x < 0 || x >= P.V) st |= SV_STATUS_BAD_TOKEN;
          else if (x != r.argmax && i < j) j = i;
        } else if (!r.accept && i < j) {
          j = i;
        }
      }
    }
    if (!(u >= 0.f && u < 1.f)) st |= SV_STATUS_BAD_UNIFORM;
    if (i0 == 0) { mine = r; tok = x; uu = u; }
  }
  if (tid == 0 && ld_dev(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
  block_or_min(st, j, sm);
  // the drawing row's record and uniform reach thread 0 through LDS
  const int ui = j < k ? k : k + 1;
  if (small && tid == j) {
    sm.dbc[0] = mine.s_t; sm.dbc[1] = mine.s_d;
    sm.f[0][0] = mine.m_t; sm.f[0][1] = mine.m_d;
    sm.bc[1] = mine.argmax;
  }
  if (small && tid == ui) sm.dbc[2] = (double)uu;
  __syncthreads();
  if (tid == 0) {
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
    GroupRec rj;
    double u;
    if (small) {
      rj.s_t = sm.dbc[0]; rj.s_d = sm.dbc[1]; rj.m_t = sm.f[0][0]; rj.m_d = sm.f[0][1]; rj.argmax = sm.bc[1];
      u = sm.dbc[2];
    } else {
      rj = ld_rec(P.grec + (int64_t)b * K1 + j);
      u = GREEDY ? 0.0 : (double)P.uniforms[(int64_t)b * (k + 2) + ui];
    }
    if (GREEDY) {
      sm.bc[2] = rj.argmax;
    } else if (!st) {
      SeqRec sr;
      sr.s_t = rj.s_t; sr.s_d = rj.s_d; sr.m_t = rj.m_t; sr.m_d = rj.m_d;
      sr.j = j; sr.valid = 1;
      sr.u = u;
      sr.resid = j < k ? 1 : 0; sr.pad = 0;
      P.srec[b] = sr;                  // read by sv_draw after this launch
    }
  }
  __syncthreads();
  for (int i = tid; i < K1; i += TPB) {
    int v = -1;
    if (!st && i < j) v = i < TPB ? tok : P.tokens[(int64_t)b * k + i];
    if (!st && i == j && GREEDY) v = sm.bc[2];
    if (st || i != j || GREEDY) P.out_tokens[(int64_t)b * K1 + i] = v;
  }
  zero_recs(P.grec + (int64_t)b * K1, K1);
  if (tid == 0) st_dev(P.sarrive + b, 0);
}

// Row combine, acceptance decision and top-32 merge of group g (run by the
// last workgroup of the group to publish), then the sequence's arrival.
template <int DT, bool GREEDY>
__device__ void group_finish(const Params &P, const Geo &G, int32_t x, Smem &sm) {
  constexpr uint32_t LOW = Fmt<DT>::LOW;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1, V = P.V;
  const int g = G.g, b = G.b, i = G.i;
  const bool pair = G.pair;
  const int nslot = nT * SLOTS, nrecw = nT * 8;

  // ---- one round of loads: candidate slots (kept in registers), tile records
  // and overflow flags (to LDS), the drafted token's logits and its uniform
  uint64_t *slots = P.cand + (int64_t)g * nslot;
  uint64_t key[KEYS_PT];
#pragma unroll
  for (int q = 0; q < KEYS_PT; ++q) {
    const int a = tid + q * TPB;
    key[q] = a < nslot ? ld_dev(slots + a) : 0ull;
  }
  const uint64_t *rsrc = (const uint64_t *)(P.recs + (int64_t)g * nT);
  uint64_t rw[RECW_PT];
#pragma unroll
  for (int q = 0; q < RECW_PT; ++q) {
    const int a = tid + q * TPB;
    rw[q] = a < nrecw ? ld_dev(rsrc + a) : 0ull;
  }
  const int32_t ov = tid < nT ? ld_dev(P.ovf + (int64_t)g * nT + tid) : 0;
  float lv = 0.f;                              // lane 0: t_x, lane 1: d_x
  float ui = 0.f;
  if (pair && wid == 0 && lane < 2 && x >= 0 && x < V) lv = load_elem<DT>(lane == 0 ? G.trow : G.drow, x);
  if (pair && tid == 0) ui = P.uniforms[(int64_t)b * (k + 2) + i];
  uint64_t *rdst = (uint64_t *)sm.m.rec;
#pragma unroll
  for (int q = 0; q < RECW_PT; ++q) {
    const int a = tid + q * TPB;
    if (a < nrecw) rdst[a] = rw[q];
  }
  {
    const uint64_t ob = __ballot(ov != 0);
    if (lane == 0 && wid < 2) sm.rescan[wid] = ob;
  }
  __syncthreads();

  // ---- wave 0: row statistics, decision, group record, and the row bound
  float M_t = NEG_INF, M_d = NEG_INF;
  double S_t = 0.0, S_d = 0.0;
  int fl = 0;
  if (wid == 0) {
    const TileRec *R = sm.m.rec;
    float am = NEG_INF, dm = NEG_INF;
    int fa = 0, fd = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + 64 * h;
      if (t < nT) { am = fmaxf(am, R[t].m_t); dm = fmaxf(dm, R[t].m_d); fa |= R[t].flags_t; fd |= R[t].flags_d; }
    }
    M_t = wave_max_f(am);
    M_d = pair ? wave_max_f(dm) : NEG_INF;
    fa = wave_or(fa);
    fd = pair ? wave_or(fd) : 0;
    if (!GREEDY) {
      double a = 0.0, d = 0.0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = lane + 64 * h;
        if (t < nT) {
          a += rescale(R[t].s_t, R[t].m_t, M_t, P.sc);
          if (pair) d += rescale(R[t].s_d, R[t].m_d, M_d, P.sc);
        }
      }
      S_t = wave_sum_d(a);
      if (pair) S_d = wave_sum_d(d);
    }
    // one data-error bit per row: NaN before +inf before an empty row
    fa = (fa & SV_STATUS_NAN) ? SV_STATUS_NAN : fa;
    fd = (fd & SV_STATUS_NAN) ? SV_STATUS_NAN : fd;
    if (!GREEDY && M_t == NEG_INF && !fa) fa = SV_STATUS_EMPTY_ROW;
    if (pair && M_d == NEG_INF && !fd) fd = SV_STATUS_EMPTY_ROW;
    fl = GREEDY ? (fa & SV_STATUS_NAN) : (fa | (pair ? fd : 0));

    if (!GREEDY) {
      // acceptance: lane 0 evaluates p_i(x_i), lane 1 q_i(x_i), side by side
      int acc = 1;
      double pv = __builtin_nan("");
      if (pair) {
        if (x < 0 || x >= V) {
          fl |= SV_STATUS_BAD_TOKEN;
          acc = 0;
        } else if (!fl) {
          const double mm = lane == 0 ? (double)M_t : (double)M_d;
          const double ss = lane == 0 ? S_t : S_d;
          pv = exp2(((double)lv - mm) * P.scd) / ss;
          const double p = readlane_d(pv, 0), q = readlane_d(pv, 1);
          const double ratio = q > 0.0 ? p / q : (p > 0.0 ? __builtin_inf() : 0.0);
          const double a = ratio < 1.0 ? ratio : 1.0;
          acc = ((double)__builtin_bit_cast(float, readlane(__float_as_uint(ui), 0)) < a) ? 1 : 0;
        } else {
          acc = 0;
        }
      }
      const double lg = log(lane == 0 ? S_t : S_d);
      if (lane == 0) {
        GroupRec gr;
        gr.s_t = S_t; gr.s_d = S_d; gr.m_t = M_t; gr.m_d = M_d;
        gr.flags = fl; gr.accept = acc; gr.argmax = -1; gr.pad = 0;
        st_rec(P.grec + g, gr);
        if (P.lse_t) P.lse_t[(int64_t)b * K1 + i] = (float)((double)M_t / (double)P.T + lg);
      }
      if (pair && lane < 2) {
        float *dst = lane == 0 ? P.p_tok : P.q_tok;
        if (dst) dst[(int64_t)b * k + i] = (float)pv;
        if (lane == 1 && P.lse_d) P.lse_d[(int64_t)b * k + i] = (float)((double)M_d / (double)P.T + lg);
      }
      // row k: tile masses of p_k for a bonus draw
      if (i == k) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = lane + 64 * h;
          if (t < nT) st_dev(P.psum + (int64_t)b * nT + t, rescale(R[t].s_t, R[t].m_t, M_t, P.sc) / S_t);
        }
      }
    }

    // the row bound rb: the 32nd largest of the tiles' lane maxima (0 when
    // there are fewer), found bit by bit from the top
    const int ntops = nT * LIST, nq = (ntops + 63) >> 6;
    uint32_t tops[TOPS_PL];
#pragma unroll
    for (int q = 0; q < TOPS_PL; ++q) {
      const int f = lane + 64 * q;
      tops[q] = (q < nq && f < ntops) ? R[f / LIST].top[f % LIST] : 0u;
    }
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 32 - Fmt<DT>::BITS; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < TOPS_PL; ++q)
        if (q < nq) cnt += __popcll(__ballot(tops[q] >= cand));
      if (cnt >= TOPK) prefix = cand;
    }
    // tiles to rescan: candidates overflowed, or the 8th lane maximum lies above
    // the bound (elements between the two were not published)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + 64 * h;
      const uint64_t sat = __ballot(t < nT && R[t].top[LIST - 1] > (prefix | LOW));
      if (lane == 0) sm.rescan[h] |= sat;
    }
    if (lane == 0) {
      sm.bc[0] = 0;
      sm.bc[1] = (int)prefix;
      sm.bc[2] = fa;                           // the target row's own flags decide its top-32
      sm.bc[6] = -1;
    }
  }
  __syncthreads();
  const uint32_t rb = (uint32_t)sm.bc[1];
  const bool nanrow = (sm.bc[2] & SV_STATUS_NAN) != 0;
  const uint64_t rs0 = sm.rescan[0], rs1 = sm.rescan[1];

  // ---- candidates at or above the bound: slots of complete tiles, then rescans
  if (!nanrow) {
#pragma unroll
    for (int q = 0; q < KEYS_PT; ++q) {
      const int a = tid + q * TPB;
      if (a < nslot && key[q]) {
        const int tc = a / SLOTS;
        const bool skip = ((tc < 64 ? rs0 >> tc : rs1 >> (tc - 64)) & 1u) != 0;
        if (!skip && (uint32_t)(key[q] >> 32) >= rb) {
          const int pos = atomicAdd(&sm.bc[0], 1);
          if (pos < MERGE_CAP) sm.m.keys[pos] = key[q];
        }
      }
    }
    for (int h = 0; h < 2; ++h) {
      uint64_t m = h ? rs1 : rs0;
      while (m) {
        const int tc = 64 * h + __builtin_ctzll(m);
        m &= m - 1;
        u32x4 r[NSEG];
        load_tile<DT>(G.trow, tc, V, P.t_vec, r);
        const int lim = V - tc * Fmt<DT>::TILE;
#pragma unroll
        for (int s = 0; s < NSEG; ++s)
#pragma unroll
          for (int w = 0; w < Fmt<DT>::W; ++w) {
            const float xv = unpack<DT>(r[s], w);
            if (tpos<DT>(s, w) < lim && xv == xv && ordered_key(xv) >= rb) {
              const int pos = atomicAdd(&sm.bc[0], 1);
              if (pos < MERGE_CAP) sm.m.keys[pos] = cand_key(xv, tc * Fmt<DT>::TILE + tpos<DT>(s, w));
            }
          }
      }
    }
  }
  __syncthreads();
  const int n = sm.bc[0];
  float *oval = P.topk_val + ((int64_t)b * K1 + i) * TOPK;
  int32_t *oidx = P.topk_idx + ((int64_t)b * K1 + i) * TOPK;
  if (nanrow) {
    for (int r = tid; r < TOPK; r += TPB) { oval[r] = __builtin_nanf(""); oidx[r] = -1; }
  } else if (n > MERGE_CAP) {
    topk_exact<DT>(G.trow, V, oval, oidx, sm);
  } else {
    for (int a = tid; a < n; a += TPB) {
      const uint64_t ka = sm.m.keys[a];
      int rank = 0;
      for (int jj = 0; jj < n; ++jj) rank += sm.m.keys[jj] > ka;
      if (rank < TOPK) {
        oidx[rank] = cand_index(ka);
        oval[rank] = cand_value(ka);
        if (rank == 0) sm.bc[6] = cand_index(ka);
      }
    }
    for (int r = n + tid; r < TOPK; r += TPB) { oval[r] = NEG_INF; oidx[r] = -1; }
    __syncthreads();
  }
  if (GREEDY && tid == 0) {
    GroupRec gr;
    gr.s_t = 0.0; gr.s_d = 0.0; gr.m_t = M_t; gr.m_d = NEG_INF;
    gr.flags = fl; gr.accept = 1; gr.argmax = sm.bc[6]; gr.pad = 0;
    st_rec(P.grec + g, gr);
  }
  const int olds = arrive(P.sarrive + b, sm);

  // every workgroup of the group has published and left: clear the group's
  // workspace (nothing in this launch reads it again)
#pragma unroll
  for (int q = 0; q < KEYS_PT; ++q) {
    const int a = tid + q * TPB;
    if (a < nslot && key[q]) st_dev(slots + a, (uint64_t)0);
  }
#pragma unroll
  for (int q = 0; q < RECW_PT; ++q) {
    const int a = tid + q * TPB;
    if (a < nrecw && rw[q]) st_dev((uint64_t *)rsrc + a, (uint64_t)0);
  }
  if (ov) st_dev(P.ovf + (int64_t)g * nT + tid, 0);
  if (tid == 0) st_dev(P.garrive + g, 0);

  if (olds < 0 || olds > k) { if (tid == 0) atomicOr(P.fault, 2); return; }  // workspace not zero-filled
  if (olds == k) seq_finish<GREEDY>(P, b, sm);
}

template <int DT, bool GREEDY>
__global__ __launch_bounds__(TPB) void sv_stream(Params P) {
  __shared__ Smem sm;
  constexpr int W = Fmt<DT>::W, TILE = Fmt<DT>::TILE;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int V = P.V;
  const int item = blockIdx.x;
  const Geo G = geo<DT, GREEDY>(P, item);
  const int c = G.c;
  const bool pair = G.pair;
  // the drafted token of a pair group (used only by the group's last workgroup)
  const int32_t xtok = pair ? P.tokens[(int64_t)G.b * P.k + G.i] : -1;

  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT>(G.trow, c, V, P.t_vec, rt);
  if (pair) load_tile<DT>(G.drow, c, V, P.d_vec, rd);
  else
#pragma unroll
    for (int s = 0; s < NSEG; ++s) rd[s] = rt[s];
  if (tid == 0) sm.bc[0] = 0;                          // candidate count

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

  // per-wave partials: max, sum relative to the wave max, flags, largest lane maxima
  {
    const float wm_t = wave_max_f(mt);
    const float wm_d = pair ? wave_max_f(md) : NEG_INF;
    const int wf_t = wave_or(ft), wf_d = pair ? wave_or(fd) : 0;
    double ws_t = 0.0, ws_d = 0.0;
    if (!GREEDY) {
      ws_t = wave_sum_d(rescale((double)st, mt, wm_t, P.sc));
      if (pair) ws_d = wave_sum_d(rescale((double)sd, md, wm_d, P.sc));
    }
    const uint32_t w8 = wave_top_list(tkey, lane);
    if (lane < LIST) sm.w8[wid * LIST + lane] = w8;
    if (lane == 0) {
      sm.f[0][wid] = wm_t; sm.f[1][wid] = wm_d; sm.i[0][wid] = wf_t; sm.i[1][wid] = wf_d;
      sm.d[0][wid] = ws_t; sm.d[1][wid] = ws_d;
    }
  }
  __syncthreads();
  // the tile's largest lane maxima (every wave derives them) and the candidate bound
  const uint32_t t8 = wave_top_list(lane < NWAVE * LIST ? sm.w8[lane] : 0u, lane);
  const uint32_t bound = readlane(t8, LIST - 1);

  // candidates: elements at or above the bound (all of a tile with fewer lanes)
  {
    const float Lf = key_value(bound);
    const int lim = V - c * TILE;                        // tile positions < lim exist
    uint32_t mask = 0;
    if (has_elem && (bound == 0u || tkey >= bound)) {
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float xv = unpack<DT>(rt[s], w);
          if (tpos<DT>(s, w) < lim && (bound == 0u || xv >= Lf)) mask |= 1u << (s * W + w);
        }
    }
    const int cnt = __popc(mask);
    if (cnt) {
      const int base = atomicAdd(&sm.bc[0], cnt);
      uint64_t *dst = P.cand + (int64_t)item * SLOTS;
      int slot = base;
      while (mask) {
        const int bit = __builtin_ctz(mask);
        mask &= mask - 1;
        const int s = bit / W, w = bit - s * W;
        if (slot < SLOTS) st_dev(dst + slot, cand_key(unpack<DT>(rt[s], w), c * TILE + tpos<DT>(s, w)));
        ++slot;
      }
      if (base + cnt > SLOTS) st_dev(P.ovf + item, 1);
    }
  }

  // the tile record (wave 0, from the four wave partials)
  if (wid == 0) {
    float m_ct = sm.f[0][0], m_cd = sm.f[1][0];
    int f_ct = sm.i[0][0], f_cd = sm.i[1][0];
    for (int w = 1; w < NWAVE; ++w) {
      m_ct = fmaxf(m_ct, sm.f[0][w]); m_cd = fmaxf(m_cd, sm.f[1][w]);
      f_ct |= sm.i[0][w]; f_cd |= sm.i[1][w];
    }
    double s_ct = 0.0, s_cd = 0.0;
    if (!GREEDY)
      for (int w = 0; w < NWAVE; ++w) {
        s_ct += rescale(sm.d[0][w], sm.f[0][w], m_ct, P.sc);
        s_cd += rescale(sm.d[1][w], sm.f[1][w], m_cd, P.sc);
      }
    TileRec r;
    r.m_t = m_ct; r.m_d = m_cd; r.s_t = s_ct; r.s_d = s_cd; r.flags_t = f_ct; r.flags_d = f_cd;
#pragma unroll
    for (int q = 0; q < LIST; ++q) r.top[q] = readlane(t8, q);
    if (lane == 0) st_rec(P.recs + item, r);
  }
  const int old = arrive(P.garrive + G.g, sm);
  if (old < 0 || old >= P.nT) { if (tid == 0) atomicOr(P.fault, 2); return; }  // workspace not zero-filled
  if (old != P.nT - 1) return;
  group_finish<DT, GREEDY>(P, G, xtok, sm);
}

// Inverse-CDF draw inside one tile: the first element (ascending index) of
// positive mass whose cumulative mass prefix + (scan base + running fp32 sum)
// exceeds tau; if rounding leaves none, the tile's last positive-mass element
// (-1 when the tile has none).  The masses are recomputed exactly as when the
// tile's total was published.
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
  first = wave_min_i(first);
  lastpos = wave_max_i(lastpos);
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

// The crossing tile of tau = u * R over the tile masses in sm.tot (tile order,
// R their sum): sm.bc[2] = the first tile whose cumulative mass exceeds tau (-1
// if none), sm.dbc[0] = the mass before it, sm.dbc[1] = tau.  Run by wave 0.
__device__ void locate_tile(int nT, double u, Smem &sm) {
  const int lane = threadIdx.x & 63;
  const double a0 = lane < nT ? sm.tot[lane] : 0.0;
  const double a1 = lane + 64 < nT ? sm.tot[lane + 64] : 0.0;
  const double c0 = wave_scan_d(a0);
  const double t0 = readlane_d(c0, 63);
  const double c1 = t0 + wave_scan_d(a1);
  const double R = readlane_d(c1, 63);
  const double tau = u * R;
  const uint64_t h0 = __ballot(lane < nT && c0 > tau), h1 = __ballot(lane + 64 < nT && c1 > tau);
  int cs = -1;
  if (h0) cs = __builtin_ctzll(h0);
  else if (h1) cs = 64 + __builtin_ctzll(h1);
  double before = 0.0;
  if (cs > 0) before = cs <= 64 ? readlane_d(c0, cs - 1) : readlane_d(c1, cs - 65);
  if (lane == 0) { sm.bc[2] = cs; sm.dbc[0] = before; sm.dbc[1] = tau; }
}

template <int DT>
__global__ __launch_bounds__(TPB) void sv_draw(Params P) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1;
  const int b = blockIdx.x / nT, c = blockIdx.x - (blockIdx.x / nT) * nT;
  const SeqRec sr = P.srec[b];
  // row k's tile masses were published for every sequence; only a bonus draw reads them
  if ((!sr.valid || sr.resid) && tid == 0) st_dev(P.psum + (int64_t)b * nT + c, 0.0);
  if (!sr.valid) return;
  const int j = sr.j;
  const bool resid = sr.resid != 0;
  const char *trow = P.target + ((int64_t)b * K1 + j) * P.tstride * Fmt<DT>::E;
  const char *drow = resid ? P.draft + ((int64_t)b * k + j) * P.dstride * Fmt<DT>::E : nullptr;
  double *masses;
  if (!resid) {
    if (c != 0) return;
    masses = P.psum + (int64_t)b * nT;
  } else {
    u32x4 rt[NSEG], rd[NSEG];
    load_tile<DT>(trow, c, P.V, P.t_vec, rt);
    load_tile<DT>(drow, c, P.V, P.d_vec, rd);
    const float mt = thread_max<DT>(rt);
    const float md = thread_max<DT>(rd);
    const float at = prob_scale(mt, sr.m_t, sr.s_t, P.sc);
    const float ad = prob_scale(md, sr.m_d, sr.s_d, P.sc);
    float seg[NSEG];
    seg_masses<DT>(rt, rd, true, mt, md, at, ad, P.sc, seg);
    double base[NSEG];
    const double tot = tile_scan(seg, base, sm);
    if (tid == 0) st_dev(P.rsum + (int64_t)b * nT + c, tot);
    const int old = arrive(P.darrive + b, sm);
    if (old < 0 || old >= nT) { if (tid == 0) atomicOr(P.fault, 2); return; }
    if (old != nT - 1) return;
    masses = P.rsum + (int64_t)b * nT;
  }

  // locate the crossing tile in tile order, then rescan it
  for (int cc = tid; cc < nT; cc += TPB) sm.tot[cc] = ld_dev(masses + cc);
  __syncthreads();
  if (wid == 0) locate_tile(nT, sr.u, sm);
  __syncthreads();
  bool use_p = false;
  if (sm.bc[2] < 0 && resid) {
    // no residual mass left (only through rounding): draw from p_j with the same uniform
    use_p = true;
    for (int cc = 0; cc < nT; ++cc) {
      const double m = tile_mass_p<DT>(P, trow, cc, sr.m_t, sr.s_t, sm);
      if (tid == 0) sm.tot[cc] = m;
    }
    __syncthreads();
    if (wid == 0) locate_tile(nT, sr.u, sm);
    __syncthreads();
  }
  const int cstar = sm.bc[2] >= 0 ? sm.bc[2] : nT - 1;
  const double prefix = sm.dbc[0], tau = sm.dbc[1];
  __syncthreads();
  const bool rmode = resid && !use_p;
  int token = tile_draw<DT>(P, trow, drow, cstar, rmode, sr.m_t, sr.s_t, sr.m_d, sr.s_d, prefix, tau, sm);
  // a tile whose recomputed masses all rounded to zero: the last positive-mass
  // element before it
  for (int cc = cstar - 1; token < 0 && cc >= 0; --cc)
    token = tile_draw<DT>(P, trow, drow, cc, rmode, sr.m_t, sr.s_t, sr.m_d, sr.s_d, 0.0, __builtin_inf(), sm);
  if (tid == 0) {
    P.out_tokens[(int64_t)b * K1 + j] = token;
    if (resid) st_dev(P.darrive + b, 0);
    SeqRec z;
    memset(&z, 0, sizeof z);
    P.srec[b] = z;
  }
  for (int cc = tid; cc < nT; cc += TPB) st_dev(masses + cc, 0.0);
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t fault, garrive, sarrive, darrive, recs, grec, srec, cand, ovf, rsum, psum, total;
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
  L.ovf = o;     o = align256(o + groups * nT * sizeof(int32_t));
  L.rsum = o;    o = align256(o + (size_t)B * nT * sizeof(double));
  L.psum = o;    o = align256(o + (size_t)B * nT * sizeof(double));
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
  P.ovf = (int32_t *)(ws + L.ovf);
  P.rsum = (double *)(ws + L.rsum);
  P.psum = (double *)(ws + L.psum);
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
