// spec_verify.hip -- speculative-sampling verification for gfx950 (MI355X).
//
// One launch of sv_verify.  Its first workgroups, one per (group, tile), stream
// the logits and assemble every sequence; in sampling mode one workgroup per
// (sequence, tile) follows and draws the residual or bonus token.
//
//  streaming  A group is, for i < k, the pair (target row i, draft row i) of a
//             sequence and, for i == k, target row k alone; in greedy mode every
//             group is one target row.  Tiles are fixed 16 KB slices of a row
//             (8192 bf16 or 4096 fp32 entries).  Each workgroup streams its
//             tile(s) once with 128-bit loads and publishes a tile record:
//               - max and sum of exp2((x - max) * log2(e)/T) of each row part
//                 (fp32 exp and per-thread fp32 sums, fp64 above the wave);
//               - 8 lane maxima of distinct lanes (a lane owns 32 bf16 or 16
//                 fp32 elements), the two largest of each wave;
//             and, as top-32 candidates, the elements at or above the smallest
//             of those 8.
//             The last tile of a group (dispatched after the others) waits for
//             the others' records and merges the group: row max and normaliser
//             in tile order, the acceptance decision, and the top-32.  The 32nd
//             largest of the tiles' lane maxima bounds the row's 32nd largest
//             element from below; candidates at or above it are ranked, and a
//             tile whose candidate threshold lies above the bound (it may hold
//             further elements above it) is rescanned, as is a tile whose
//             candidates overflowed their slots.  The group record (offsets of
//             the row's log-normaliser, flags, decision) goes out as soon as
//             the decision is made; each of its words is never 0 once written
//             (the offsets word stored complemented), so a draw or the
//             assembly that reads them nonzero has the record.
//             The merge of row k (dispatched after rows 0..k-1) waits for the
//             sequence's other groups and assembles it: the first rejection j
//             (greedy: the first draft that differs from the argmax), the
//             tokens, and whether the sequence has a data error.
//  draw       The draw workgroups of a sequence learn the drawing row from the
//             group records as soon as it is decided: pair row j after a
//             rejection (residual max(0, p - q)), row k after k acceptances
//             (p).  For a residual each publishes one tile's total mass; once
//             all tiles of the row are in, every one finds the crossing tile of
//             u * R over the totals in tile order, and the one that holds it
//             draws the token from its registers.  For the bonus row the tile
//             masses follow from the row's streaming statistics, so only the
//             workgroup of the crossing tile reads its elements.
//
// A streaming workgroup only ever waits for workgroups of lower items, which
// its XCD dispatches first (items run in order within an XCD; a group or a
// sequence that spans two XCDs waits across the boundary, a handful of
// workgroups at most); a draw workgroup waits for streaming workgroups and for
// the other draw workgroups of its sequence, dispatched with it.  Every
// wait is bounded in time: a wait that gives up sets the fault word (reported
// as SV_STATUS_SYNC_TIMEOUT) and the kernel still finishes.  Data moves
// between workgroups through the workspace with device-scope write-through
// stores and device-scope loads, ordered by waiting for the stores to complete
// before the counter or flag that announces them is written, or as words that
// are never 0 once written, which the reader reads again until they are (tile
// records and candidate slots in the base bf16 sampling build, group records
// in sampling mode, tile totals).  Wave-level
// reductions and scans run on DPP row shifts and broadcasts in a fixed order,
// so every reduction is deterministic.
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
#include <type_traits>

#include "spec_verify.h"
#include "sv_device.h"
#include "sv_host.h"

namespace {

using namespace sv_dev;

constexpr int LIST = 8;                // lane maxima a tile record keeps
constexpr int SLOTS = 32;              // candidate slots per tile
constexpr int MERGE_CAP = 512;         // candidates a row merge ranks in LDS
constexpr int STAGE = 128;             // candidates a tile stages in LDS (its top SLOTS are published)
constexpr int STAGE_V = 128;           // vectors holding candidates a tile stages in LDS
constexpr int TOPK = SV_TOPK;
constexpr int MAX_TILES = 64;          // tiles per row: one merge lane each
// The streaming loads are marked nontemporal for fp32 logits only: with bf16
// logits ordinary loads measured faster on MI355X (0.5-1.3 us per step at
// B = 1..256, k = 3..8), with fp32 logits nontemporal ones (7 us per step at
// B = 32, k = 15).
template <int DT> constexpr bool kStreamNT = DT == SV_F32;
// Waves per SIMD the kernel is built for: 8 for fp32 (64 VGPRs; at B = 32,
// k = 15 greedy 83.6 -> 80.3 us, sampling 135.6 -> 132.6 us against 6).  bf16
// has two builds, chosen per shape by the measured table: the format's budget
// (6 waves, 80 VGPRs) and a high-occupancy one (8 waves, 64 VGPRs), which
// keeps more workgroups resident at large batches but measured slower at small
// ones.  No build uses scratch memory; the SGPRs the compiler spills (kernel
// arguments, mostly) go to VGPR lanes.
template <int DT, bool GREEDY, bool HI> constexpr int kWaves =
    DT == SV_F32 ? 8 : (HI ? 8 : Fmt<DT>::WAVES);
constexpr int KEYS_PT = MAX_TILES * SLOTS / TPB;   // candidate slots per merge thread
// How a group's merge learns that its tiles' records and candidate slots are
// out.  Counted: each tile waits for its stores and bumps the group's
// counter, and the merge waits for the count, then loads records and slots in
// one round.  Uncounted: the merge reads the records as they land (their
// words, stored complemented, are never 0 once written), decides, and only
// then reads the slots each record says are in use, again until written.
// Uncounted is the base bf16 sampling build's (steady B = 32, k = 3: 29.0 ->
// 28.0 us; B = 1..4, k = 8: 0.7-0.9 us less); counted measured faster for fp32
// (wide: 112.6 against 119.5 us), in greedy mode, whose decision needs the
// top-32 (wide greedy: 64.1 against 71.6 us), and for the high-occupancy
// build's large batches (B = 256, k = 3: 124.0 against 124.6 us).
template <int DT, bool GREEDY, bool HI> constexpr bool Uncounted = DT == SV_BF16 && !GREEDY && !HI;
// Published per (group, tile) by the stream workgroups; 8 words, stored as
// their complements by the uncounted build (see Uncounted).
struct TileRec {
  float m_t, m_d;          // tile max of the target / draft row part
  double s_t, s_d;         // sum exp2((x - m) * sc) over the tile part
  int32_t flags;           // SV_STATUS_* bits: target row part | draft row part << 8 (bits
                           // 0-15), candidate slots in use (16-23), overflow: rescan the tile (24)
  uint32_t kthr;           // ordered key of the candidate threshold (0: every element)
  uint32_t top[LIST];      // ordered keys of 8 lane maxima of distinct lanes, the two
                           // largest of each wave (0: no lane)
};
static_assert(sizeof(TileRec) == 64, "tile record");

// Published per group by its merging workgroup.
struct GroupRec {
  float ot, od;            // sampling: offsets m * log2(e)/T + log2(s) of the target / draft row,
                           // stored as the complement of their bits (never 0 once written)
  int32_t flags;           // SV_STATUS_* bits of this group's rows and token
  int32_t argmax;          // greedy: top-1 index of the target row
  int32_t accept;          // 1 when the drafted token passed (pair groups)
  int32_t ready;           // sampling: 1, written with the rest (the offsets word validates itself)
};
static_assert(sizeof(GroupRec) == 24, "group record");

// Written by the sequence assembly for the draw workgroups.
struct SeqRec {
  int32_t j;               // first rejection (k: none)
  int32_t state;           // 0: not assembled yet; 1: assembled; 2: a data error, nothing to draw
};
constexpr int SREC_STRIDE = 256;       // bytes per sequence record: its pollers share no line

struct Params {
  const char *target, *draft;
  int64_t tstride, dstride;            // row strides in elements
  const int32_t *tokens;
  const float *uniforms;
  int32_t *accepted_len, *out_tokens, *topk_idx, *status;
  float *topk_val, *lse_t, *lse_d, *p_tok, *q_tok;
  int32_t *fault;                      // bit 1: a wait gave up; bit 2: workspace not zero-filled
  int32_t *garrive, *sarrive, *ddone;          // counters, CTR int32 apart
  TileRec *recs;
  GroupRec *grec;
  SeqRec *srec;
  uint64_t *cand;                      // [group][tile][SLOTS] candidate keys, 0 = empty
  uint64_t *dtot;                      // [sequence][tile][2] drawing-row tile totals (residual, p) as
                                       // tot_word: 0 until published
  int32_t B, k, V, nT;
  int32_t items;                       // streaming workgroups: B * (k + 1) * nT
  int32_t xcd_runs;                    // 1: one contiguous run of items per XCD; 0: launch order
  float T, sc;                         // sc = log2(e) / T
  double scd;
  int32_t t_vec, d_vec;                // rows 16-byte aligned
};

struct Smem {
  union {
    uint64_t keys[MERGE_CAP];          // row merge: the candidates at or above the bound
    struct {                           // exact top-32 fallback
      uint32_t hist[2048];
      int32_t part[TPB];
      uint64_t list[TOPK];
    } fb;
    struct {                           // draw: the crossing thread's elements
      uint32_t t[NSEG * 4], d[NSEG * 4];
    } walk;
    struct {                           // stream: vectors that hold candidates, then the candidates
      u32x4 v[STAGE_V];                // raw vector
      int32_t pos[STAGE_V];            // tile position of its first element
      uint64_t ck[STAGE];              // candidates: value bits and tile position, then keys
    } st;
  };
  uint32_t w8[LIST];                   // stream: each wave's two largest lane maxima
  float f[4][NWAVE];
  int32_t i[4][NWAVE];
  double d[4][NWAVE];
  int32_t bc[8];
  double dbc[8];
  uint64_t rescan;                     // row merge: tiles to rescan
  int32_t i4[MAX_TILES];               // row merge: each tile's candidate slots in use
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
// A staged candidate before its key is formed: value bits and tile position.
__device__ __forceinline__ uint64_t raw_cand(float v, int pos) {
  return ((uint64_t)__float_as_uint(v) << 32) | (uint32_t)pos;
}
__device__ __forceinline__ uint64_t key_of_raw(uint64_t r, int x0) {
  return cand_key(__uint_as_float((uint32_t)(r >> 32)), x0 + (int)(uint32_t)r);
}
__device__ __forceinline__ int32_t cand_index(uint64_t k) { return (int32_t)(0xfffffu - ((uint32_t)k >> 1)); }
__device__ __forceinline__ float cand_value(uint64_t k) {
  return (k & 1u) ? -0.0f : key_value((uint32_t)(k >> 32));
}

// The two largest keys of the wave's lanes (equal keys of different lanes
// count twice; 0 where fewer lanes hold a nonzero key), in every lane.
__device__ __forceinline__ void wave_top2(uint32_t key, uint32_t &k1, uint32_t &k2) {
  uint32_t a = key, c = 0u;
#define SV_TOP2_STEP(CTRL, RM, BM)                                   \
  {                                                                   \
    const uint32_t b = dpp<CTRL, RM, BM>(0u, a), d = dpp<CTRL, RM, BM>(0u, c); \
    const uint32_t hi = a > b ? a : b, lo = a > b ? b : a;           \
    c = lo > c ? lo : c;                                              \
    c = d > c ? d : c;                                                \
    a = hi;                                                           \
  }
  SV_TOP2_STEP(0x111, 0xf, 0xf)
  SV_TOP2_STEP(0x112, 0xf, 0xf)
  SV_TOP2_STEP(0x114, 0xf, 0xe)
  SV_TOP2_STEP(0x118, 0xf, 0xc)
  SV_TOP2_STEP(0x142, 0xa, 0xf)
  SV_TOP2_STEP(0x143, 0xc, 0xf)
#undef SV_TOP2_STEP
  k1 = readlane(a, 63);
  k2 = readlane(c, 63);
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

// A sampling group record, read word by word until each is nonzero (each is
// never 0 once written); bounded, as every wait.
__device__ __forceinline__ GroupRec poll_rec(const GroupRec *src, int32_t *fault) {
  const uint64_t *s = (const uint64_t *)src;
  uint64_t w[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) w[q] = ld_dev(s + q);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (!w[0] || !w[1] || !w[2]) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
      atomicOr(fault, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (!w[q]) w[q] = ld_dev(s + q);
  }
  GroupRec r;
  __builtin_memcpy(&r, w, sizeof(r));
  return r;
}

// Sequence assembly (run by the merge of row k once the sequence's other
// groups have published): status, first rejection j, and the tokens; greedy
// emits everything, sampling leaves the drawn token to the draw workgroups.
template <int DT, bool GREEDY>
__device__ __forceinline__ void seq_finish(const Params &P, int b, Smem &sm) {
  const int tid = threadIdx.x;
  const int k = P.k, K1 = k + 1;
  const bool small = k + 2 <= TPB;           // one entry per thread: no reloads
  // one round of loads: group records, drafted tokens, uniforms, the fault word
  int st = 0, j = k;
  GroupRec mine = {};
  int32_t tok = 0;
  for (int i0 = 0; i0 < k + 2; i0 += TPB) {
    const int i = i0 + tid;
    GroupRec r = {};
    if (i < K1) r = GREEDY ? ld_rec(P.grec + (int64_t)b * K1 + i) : poll_rec(P.grec + (int64_t)b * K1 + i, P.fault);
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
    if (i0 == 0) { mine = r; tok = x; }
  }
  if (tid == 0 && ld_dev(P.fault)) st |= SV_STATUS_SYNC_TIMEOUT;
  block_or_min(st, j, sm);
  // greedy: the argmax of row j reaches every thread through LDS
  if (GREEDY) {
    if (small && tid == j) sm.bc[1] = mine.argmax;
    if (!small && tid == 0) sm.bc[1] = ld_rec(P.grec + (int64_t)b * K1 + j).argmax;
    __syncthreads();
  }
  const int amax = GREEDY ? sm.bc[1] : -1;
  if (tid == 0) {
    if (P.status) P.status[b] = st;
    P.accepted_len[b] = st ? -1 : j;
  }
  for (int i = tid; i < K1; i += TPB) {
    int v = -1;
    if (!st && i < j) v = i < TPB ? tok : P.tokens[(int64_t)b * k + i];
    if (!st && i == j && GREEDY) v = amax;
    if (st || i != j || GREEDY) P.out_tokens[(int64_t)b * K1 + i] = v;
  }
  if (GREEDY) {
    zero_recs(P.grec + (int64_t)b * K1, K1);
  } else if (tid == 0) {
    // the draw workgroups read the group records until they finish, and clear them
    // j and the state go out in one 64-bit store: a reader that sees the
    // state sees j, with no wait between the two
    SeqRec *rec = (SeqRec *)((char *)P.srec + (int64_t)b * SREC_STRIDE);
    st_dev((uint64_t *)rec, ((uint64_t)(uint32_t)(st ? 2 : 1) << 32) | (uint32_t)j);
  }
}

// 2^a for a <= 0 to about 2e-7 relative: the integer part scales exactly, the
// fraction in [-1/2, 1/2] goes through the hardware fp32 exp2
__device__ __forceinline__ double exp2_split(double a) {
  if (!(a > -1100.0)) return 0.0;
  const double n = __builtin_rint(a);
  return __builtin_ldexp((double)__builtin_amdgcn_exp2f((float)(a - n)), (int)n);
}

// log2 of s > 0 to about 1e-7 absolute: exponent exactly, mantissa in
// [1/2, 1) through the hardware fp32 log2
__device__ __forceinline__ double log2_split(double s) {
  int e;
  const double m = __builtin_frexp(s, &e);
  return (double)e + (double)__builtin_amdgcn_logf((float)m);
}
__device__ __forceinline__ double log_split(double s) { return log2_split(s) * 0.6931471805599453; }

// A tile's statistics from its waves' entries in LDS: maxima, flags and, in
// sampling mode, the exp sums rescaled to the tile maxima in wave order.
struct TileStats {
  float m_t, m_d;
  int f_t, f_d;
  double s_t, s_d;
};
template <bool GREEDY> __device__ __forceinline__ TileStats tile_stats(const Smem &sm, float sc) {
  TileStats r;
  r.m_t = sm.f[0][0]; r.m_d = sm.f[1][0];
  r.f_t = sm.i[0][0]; r.f_d = sm.i[1][0];
  for (int w = 1; w < NWAVE; ++w) {
    r.m_t = fmaxf(r.m_t, sm.f[0][w]); r.m_d = fmaxf(r.m_d, sm.f[1][w]);
    r.f_t |= sm.i[0][w]; r.f_d |= sm.i[1][w];
  }
  r.s_t = 0.0; r.s_d = 0.0;
  if (!GREEDY)
    for (int w = 0; w < NWAVE; ++w) {
      r.s_t += rescale(sm.d[0][w], sm.f[0][w], r.m_t, sc);
      r.s_d += rescale(sm.d[1][w], sm.f[1][w], r.m_d, sc);
    }
  return r;
}
// Words 0-2 of a tile record (maxima; target sum; draft sum), NaN canonical
// in the uncounted build so that the complement of a word is never 0.
template <bool UNC> __device__ __forceinline__ uint64_t stat_word(const TileStats &t, int q) {
  auto canon_f = [](float v) { return !UNC || v == v ? __float_as_uint(v) : 0x7fc00000u; };
  auto canon_d = [](double v) { return !UNC || v == v ? __builtin_bit_cast(uint64_t, v) : 0x7ff8000000000000ull; };
  return q == 0 ? ((uint64_t)canon_f(t.m_d) << 32) | canon_f(t.m_t) : canon_d(q == 1 ? t.s_t : t.s_d);
}

// Row combine, acceptance decision and top-32 merge of group g (run by its last
// tile once the others have published), then the sequence's arrival.
template <int DT, bool GREEDY, bool HI>
__device__ __forceinline__ void group_finish(const Params &P, const Geo &G, int32_t x, Smem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1, V = P.V;
  const int g = G.g, b = G.b, i = G.i;
  const bool pair = G.pair;
  const int nslot = nT * SLOTS;

  // ---- one round of loads: tile records (wave 0, lane t: tile t), the
  // drafted token's logits and uniform, and, in counted mode, the candidate
  // slots (all threads).  Record words are stored complemented and are never
  // 0 once written: in uncounted mode waves 0 and 1 read a word again until
  // it is (a tile's record goes out after its slots)
  constexpr bool UNC = Uncounted<DT, GREEDY, HI>;
  uint64_t *slots = P.cand + (int64_t)g * nslot;
  uint64_t key[KEYS_PT];
  if (!UNC) {
#pragma unroll
    for (int q = 0; q < KEYS_PT; ++q) {
      const int a = tid + q * TPB;
      key[q] = a < nslot ? ld_dev(slots + a) : 0ull;
    }
  }
  // wave 0 takes words 0-3 of tile record `lane` (statistics), wave 1 words
  // 3-7 (candidate threshold, slots used, overflow, lane maxima)
  uint64_t *rsrc = (uint64_t *)(P.recs + (int64_t)g * nT) + lane * 8;
  uint64_t rw[8];
  const bool own = wid == 0 && lane < nT, own1 = wid == 1 && lane < nT;
  auto mine = [&](int q) { return (own && q <= 3) || (own1 && q >= 3); };
#pragma unroll
  for (int q = 0; q < 8; ++q) rw[q] = mine(q) ? ld_dev(rsrc + q) : ~0ull;
  float lv = 0.f;                              // lane 0: t_x, lane 1: d_x
  float ui = 0.f;
  if (pair && wid == 0 && lane < 2 && x >= 0 && x < V) lv = load_elem<DT>(lane == 0 ? G.trow : G.drow, x);
  if (pair && tid == 0) ui = P.uniforms[(int64_t)b * (k + 2) + i];
  if (UNC && wid < 2) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      bool miss = false;
#pragma unroll
      for (int q = 0; q < 8; ++q) miss |= rw[q] == 0ull;
      if (!__ballot(miss)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
        if (lane == 0) atomicOr(P.fault, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (rw[q] == 0ull) rw[q] = ld_dev(rsrc + q);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) rw[q] = mine(q) ? (UNC ? ~rw[q] : rw[q]) : 0ull;
  // wave 1: each tile's slots in use, for the uncounted slot reads after the decision
  if (UNC && own1) sm.i4[lane] = (int)((uint32_t)rw[3] >> 16 & 0xffu);

  // ---- wave 0: row statistics, decision and group record; wave 1: the row bound
  float M_t = NEG_INF;
  int fl = 0;
  if (wid == 0) {
    const float tm_t = __uint_as_float((uint32_t)rw[0]), tm_d = __uint_as_float((uint32_t)(rw[0] >> 32));
    const double ts_t = __builtin_bit_cast(double, rw[1]), ts_d = __builtin_bit_cast(double, rw[2]);
    int fa = own ? (int)((uint32_t)rw[3] & 0xffu) : 0, fd = own ? (int)(((uint32_t)rw[3] >> 8) & 0xffu) : 0;
    M_t = wave_max_f(own ? tm_t : NEG_INF);
    const float M_d = pair ? wave_max_f(own ? tm_d : NEG_INF) : NEG_INF;
    fa = wave_or(fa);
    fd = pair ? wave_or(fd) : 0;
    double S_t = 0.0, S_d = 0.0;
    if (!GREEDY) {
      S_t = wave_sum_d(own ? rescale(ts_t, tm_t, M_t, P.sc) : 0.0);
      if (pair) S_d = wave_sum_d(own ? rescale(ts_d, tm_d, M_d, P.sc) : 0.0);
    }
    // one data-error bit per row: NaN before +inf before an empty row
    fa = (fa & SV_STATUS_NAN) ? SV_STATUS_NAN : fa;
    fd = (fd & SV_STATUS_NAN) ? SV_STATUS_NAN : fd;
    if (!GREEDY && M_t == NEG_INF && !fa) fa = SV_STATUS_EMPTY_ROW;
    if (pair && M_d == NEG_INF && !fd) fd = SV_STATUS_EMPTY_ROW;
    fl = GREEDY ? (fa & SV_STATUS_NAN) : (fa | (pair ? fd : 0));

    if (!GREEDY) {
      // acceptance: lane 0 evaluates e_p = 2^((t_x - m_t) sc), lane 1 e_q for
      // the draft, side by side; p = e_p / s_t and q = e_q / s_d, and u < min(1,
      // p / q) is tested as u < 1 and u e_q s_t < e_p s_d (q = 0: p > 0), with
      // no division on the way to the group record
      int acc = 1;
      double ev = __builtin_nan("");
      if (pair) {
        if (x < 0 || x >= V) {
          fl |= SV_STATUS_BAD_TOKEN;
          acc = 0;
        } else if (!fl) {
          const double mm = lane == 0 ? (double)M_t : (double)M_d;
          ev = exp2_split(((double)lv - mm) * P.scd);
          const double ep = readlane_d(ev, 0), eq = readlane_d(ev, 1);
          const double u = (double)__uint_as_float(readlane(__float_as_uint(ui), 0));
          acc = (u < 1.0 && (eq > 0.0 ? u * eq * S_t < ep * S_d : ep > 0.0)) ? 1 : 0;
        } else {
          acc = 0;
        }
      }
      if (lane == 0) {
        GroupRec gr;
        gr.ot = (float)((double)M_t * P.scd + log2_split(S_t));
        gr.od = pair ? (float)((double)M_d * P.scd + log2_split(S_d)) : 0.f;
        gr.ot = __uint_as_float(~__float_as_uint(gr.ot == gr.ot ? gr.ot : __builtin_nanf("")));
        gr.od = __uint_as_float(~__float_as_uint(gr.od == gr.od ? gr.od : __builtin_nanf("")));
        gr.flags = fl; gr.argmax = -1; gr.accept = acc; gr.ready = 1;
        st_rec(P.grec + g, gr);
      }
      // the aux outputs, after the record
      const double lg = log_split(lane == 0 ? S_t : S_d);
      if (lane == 0 && P.lse_t) P.lse_t[(int64_t)b * K1 + i] = (float)((double)M_t / (double)P.T + lg);
      if (pair && lane < 2) {
        float *dst = lane == 0 ? P.p_tok : P.q_tok;
        if (dst) dst[(int64_t)b * k + i] = (float)(ev / (lane == 0 ? S_t : S_d));
        if (lane == 1 && P.lse_d) P.lse_d[(int64_t)b * k + i] = (float)((double)M_d / (double)P.T + lg);
      }
      // the group record is out, ready flag included, with no wait for its
      // stores: each of its three words is never 0 once written (the offsets
      // complemented, argmax -1 beside the flags, ready beside accept), so the
      // draws and the sequence's assembly read a word again until it is
      // nonzero.  (The top-32 is not part of it.)
    }

    if (lane == 0) {
      sm.bc[2] = fa;                           // the target row's own flags decide its top-32
      sm.bc[6] = -1;
    }
  } else if (wid == 1) {
    // the row bound rb: the 32nd largest of the tiles' lane maxima on 16-bit
    // buckets (0 when there are fewer than 32), found bit by bit from the top
    const uint32_t kthr = (uint32_t)(rw[3] >> 32);
    uint32_t top[LIST];
#pragma unroll
    for (int q = 0; q < LIST / 2; ++q) {
      top[2 * q] = (uint32_t)rw[4 + q];
      top[2 * q + 1] = (uint32_t)(rw[4 + q] >> 32);
    }
    uint32_t rb = 0;
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t c = rb | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < LIST; ++q) cnt += top[q] >= c ? 1 : 0;
      if (wave_sum_i(cnt) >= TOPK) rb = c;
    }
    // tiles to rescan: candidates overflowed, or the candidate threshold lies
    // above the bound (elements between the two were not published)
    const bool ov = ((uint32_t)rw[3] >> 24 & 1u) != 0;
    const uint64_t rs = __ballot(own1 && (ov || kthr > (rb | Fmt<DT>::LOW)));
    if (lane == 0) {
      sm.rescan = rs;
      sm.bc[5] = 0;
      sm.bc[1] = (int)rb;
    }
  }
  __syncthreads();
  const uint32_t rb = (uint32_t)sm.bc[1];
  const bool nanrow = (sm.bc[2] & SV_STATUS_NAN) != 0;
  const uint64_t rs = sm.rescan;
  // uncounted: the candidate slots in use (each tile's count came with its
  // record), read now, so that in row k's merge they arrive while the
  // sequence is assembled; a slot that reads 0 is read again until written
  // (the thread index passes through an empty asm: recomputing the slot
  // indices costs less than keeping them live).  Counted: the slots that hold
  // a key (to clear them at the end), so that the keys themselves are dead
  // across the rescans below
  uint32_t kheld = 0;
  int tid2 = tid;
  if (UNC) asm volatile("" : "+v"(tid2));
  if (UNC) {
#pragma unroll
    for (int q = 0; q < KEYS_PT; ++q) {
      const int a = tid2 + q * TPB;
      const bool want = a < nslot && (a & (SLOTS - 1)) < sm.i4[a / SLOTS];
      kheld |= want ? 1u << q : 0u;
      key[q] = want ? ld_dev(slots + a) : 0ull;
    }
  }
  // sampling: the sequence's assembly needs no top-32, so row k assembles
  // the sequence (reading the group records as they land) before its own merge
  if (!GREEDY && i == k) seq_finish<DT, GREEDY>(P, b, sm);
  if (UNC) {
    if (kheld) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        bool miss = false;
#pragma unroll
        for (int q = 0; q < KEYS_PT; ++q) miss |= ((kheld >> q) & 1u) && key[q] == 0ull;
        if (!miss) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
          atomicOr(P.fault, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int q = 0; q < KEYS_PT; ++q)
          if (((kheld >> q) & 1u) && key[q] == 0ull) key[q] = ld_dev(slots + tid2 + q * TPB);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < KEYS_PT; ++q) kheld |= key[q] ? 1u << q : 0u;
  }

  // ---- candidates at or above the bound: slots of complete tiles, then rescans
  if (!nanrow) {
    int tid3 = tid;
    if (UNC) asm volatile("" : "+v"(tid3));
#pragma unroll
    for (int q = 0; q < KEYS_PT; ++q) {
      const int a = tid3 + q * TPB;
      if (a < nslot && key[q] && !((rs >> (a / SLOTS)) & 1u) && (uint32_t)(key[q] >> 32) >= rb) {
        const int pos = atomicAdd(&sm.bc[5], 1);
        if (pos < MERGE_CAP) sm.keys[pos] = key[q];
      }
    }
    // (a rescanned tile is read in two halves of NSEG / 2 vectors per thread,
    // which keeps this rare path within the streaming path's registers)
    constexpr int HS = NSEG / 2, HALF = TPB * HS * Fmt<DT>::W;
    uint64_t m = rs;
    while (m) {
      const int tc = __builtin_ctzll(m);
      m &= m - 1;
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        u32x4 r[HS];
        load_tile<DT, false, HS, kStreamNT<DT>>(G.trow, 2 * tc + h, V, P.t_vec, r);
        const int x0 = tc * Fmt<DT>::TILE + h * HALF;
#pragma unroll
        for (int s = 0; s < HS; ++s)
#pragma unroll
          for (int w = 0; w < Fmt<DT>::W; ++w) {
            const float xv = unpack<DT>(r[s], w);
            const int x = x0 + tpos<DT>(s, w);
            if (x < V && xv == xv && ordered_key(xv) >= rb) {
              const int pos = atomicAdd(&sm.bc[5], 1);
              if (pos < MERGE_CAP) sm.keys[pos] = cand_key(xv, x);
            }
          }
      }
    }
  }
  __syncthreads();
  const int n = sm.bc[5];
  float *oval = P.topk_val + ((int64_t)b * K1 + i) * TOPK;
  int32_t *oidx = P.topk_idx + ((int64_t)b * K1 + i) * TOPK;
  if (nanrow) {
    for (int r = tid; r < TOPK; r += TPB) { oval[r] = __builtin_nanf(""); oidx[r] = -1; }
  } else if (n > MERGE_CAP) {
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
    __syncthreads();
  }
  if (GREEDY && tid == 0) {
    GroupRec gr;
    gr.ot = 0.f; gr.od = 0.f;
    gr.flags = fl; gr.argmax = sm.bc[6]; gr.accept = 1; gr.ready = 0;
    st_rec(P.grec + g, gr);
  }
  // greedy: announce the group record once thread 0's stores of it have
  // completed.  Then clear the group's workspace: nothing in this launch reads
  // it again, so no wave waits for these stores (waiting for all of the
  // merge's stores measured ~5 us slower per step at B = 256, k = 3)
  if (GREEDY && wid == 0) {
    stores_done();
    if (i != k && tid == 0) add_dev_noret(P.sarrive + (int64_t)b * CTR, 1);
  }
  int tid4 = tid;
  if (UNC) asm volatile("" : "+v"(tid4));
#pragma unroll
  for (int q = 0; q < KEYS_PT; ++q) {
    const int a = tid4 + q * TPB;
    if ((kheld >> q) & 1u) st_dev(slots + a, (uint64_t)0);
  }
  if (own) {
    // (sampling: row k's maximum and sum words stay for a bonus draw; the
    // sequence's last draw workgroup clears them)
    const int q0 = !GREEDY && i == k ? 2 : 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q >= q0) st_dev(rsrc + q, (uint64_t)0);
  }
  if (!GREEDY || i != k) return;
  // row k is the sequence's last group: wait for the others, then assemble
  if (tid == 0) {
    const int v = wait_at_least(P.sarrive + (int64_t)b * CTR, k, P.fault);
    if (v > k) atomicOr(P.fault, 2);                                 // workspace not zero-filled
    st_dev(P.sarrive + (int64_t)b * CTR, 0);
  }
  __syncthreads();
  seq_finish<DT, GREEDY>(P, b, sm);
}

// The thread's elements of one tile row as fp32, vector by vector.
template <int DT> struct Elems {
  float x[NSEG][Fmt<DT>::W];
};
template <int DT> __device__ __forceinline__ void unpack_all(const u32x4 (&r)[NSEG], Elems<DT> &e) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) e.x[s][w] = unpack<DT>(r[s], w);
}
// Vector s of a thread's elements packed again as loaded (bf16: the high
// halves of two fp32 values per word; fp32: the bits).
template <int DT> __device__ __forceinline__ u32x4 repack(const Elems<DT> &e, int s) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (DT == SV_BF16)
      v[q] = __builtin_amdgcn_perm(__float_as_uint(e.x[s][2 * q + 1]), __float_as_uint(e.x[s][2 * q]), 0x07060302u);
    else
      v[q] = __float_as_uint(e.x[s][q]);
  }
  return v;
}
template <int DT> __device__ __forceinline__ float vmax_of(const Elems<DT> &e, int s) {
  float m = e.x[s][0];
#pragma unroll
  for (int w = 1; w < Fmt<DT>::W; ++w) m = fmax_nan(m, e.x[s][w]);
  return m;
}
template <int DT> __device__ __forceinline__ bool has_nan_of(const Elems<DT> &e) {
  bool nan = false;
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) nan |= !(e.x[s][w] == e.x[s][w]);
  return nan;
}

// Wave statistics of one row part: the wave max wm and the sum of
// exp2((x - wm) * sc) over the wave's elements (fp32 per thread and wave,
// returned in fp64 with the rounding of wm * sc corrected); flags NaN / +inf.
template <int DT>
__device__ __forceinline__ void wave_stats(const Elems<DT> &e, float mt, float sc, float &wm, double &ws, int &flags) {
  wm = wave_max_f(mt);
  const float ref = wm == NEG_INF ? 0.f : wm;
  const float chi = ref * sc, clo = fmaf(ref, sc, -chi);    // ref * sc = chi + clo exactly
  float st = 0.f;
#pragma unroll
  for (int g = 0; g < NSEG; ++g)
#pragma unroll
    for (int w = 0; w < Fmt<DT>::W; ++w) st += __builtin_amdgcn_exp2f(fmaf(e.x[g][w], sc, -chi));
  const bool bad = !(st == st);
  flags = 0;
  if (__ballot(bad)) flags = __ballot(bad && has_nan_of<DT>(e)) ? SV_STATUS_NAN : SV_STATUS_POSINF;
  // exp2(x*sc - ref*sc) = exp2(x*sc - chi) * exp2(-clo), |clo| <= ulp(chi) / 2
  ws = (double)wave_sum_f(st) * (1.0 - (double)clo * 0.69314718055994531);
}

// Mass of element w of a vector: max(0, p - q) in residual mode, else p, with
// p = exp2(x * sc - ot) and q = exp2(y * sc - od), where ot = m_t * sc +
// log2(s_t) folds the row max and normaliser into one offset (od likewise).
__device__ __forceinline__ float mass_of(float x, float y, bool rmode, float ot, float od, float sc) {
  const float p = __builtin_amdgcn_exp2f(fmaf(x, sc, -ot));
  if (!rmode) return p;
  const float r = p - __builtin_amdgcn_exp2f(fmaf(y, sc, -od));
  return r > 0.f ? r : 0.f;
}
template <int DT>
__device__ __forceinline__ float draw_mass(const u32x4 &vt, const u32x4 &vd, int w, bool rmode, float ot, float od,
                                           float sc) {
  return mass_of(unpack<DT>(vt, w), unpack<DT>(vd, w), rmode, ot, od, sc);
}

// Element e of a thread's draw-order elements, held as 32-bit words.
template <int DT> __device__ __forceinline__ float elem_of_words(const uint32_t *words, int e) {
  if constexpr (DT == SV_BF16) {
    const uint32_t word = words[e >> 1];
    return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
  } else {
    return __uint_as_float(words[e]);
  }
}

// The draw in the workgroup whose tile holds the crossing: thread t's own
// mass `mine` and the mass `base` of the tile's elements before it, the tile's
// elements rt (and rd for a residual) in registers, the mass before the tile
// and tau in sm.dbc[0..1].
template <int DT>
__device__ __forceinline__ void draw_crossing(const Params &P, int b, int c, int j, const u32x4 (&rt)[NSEG],
                                              const u32x4 (&rd)[NSEG], bool rmode, float ot, float od, float mine,
                                              double base, SeqRec *rec, Smem &sm) {
  constexpr int W = Fmt<DT>::W;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K1 = P.k + 1;
  // this tile holds the crossing.  Running totals only grow along a
  // thread's elements, so the first element past tau lies in the first
  // thread whose total passes it (should rounding leave no element past
  // tau: the tile's last positive-mass element, in the last thread with
  // mass).  That thread hands its elements to wave 0, whose lanes compute
  // one mass each and form the thread's running totals in its own order,
  // so the last of them equals its total bit for bit.
  const double prefix = sm.dbc[0], tau = sm.dbc[1];
  const bool past = mine > 0.f && prefix + (base + (double)mine) > tau;
  const int tfirst = wave_min_i(past ? tid : 0x7fffffff);
  const int tlast = wave_max_i(mine > 0.f ? tid : -1);
  if (lane == 0) { sm.i[2][wid] = tfirst; sm.i[3][wid] = tlast; }
  __syncthreads();
  int tf = sm.i[2][0], tl = sm.i[3][0];
  for (int w = 1; w < NWAVE; ++w) {
    tf = sm.i[2][w] < tf ? sm.i[2][w] : tf;
    tl = sm.i[3][w] > tl ? sm.i[3][w] : tl;
  }
  const int walker = tf != 0x7fffffff ? tf : tl;
  if (tid == walker) {
#pragma unroll
    for (int s = 0; s < NSEG; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) { sm.walk.t[s * 4 + q] = rt[s][q]; sm.walk.d[s * 4 + q] = rd[s][q]; }
    sm.dbc[3] = base;
  }
  __syncthreads();
  if (wid == 0) {
    constexpr int NE = NSEG * W;                     // elements per thread (<= 64)
    // the assembly's state (the token stands unless it found a data error),
    // read while the walk below runs (by every lane: one request, and no
    // lane mask that would make the compiler wait for it at once)
    int state = ld_dev(&rec->state);
    int pos = -1;
    if (walker >= 0) {
      const float m = lane < NE ? mass_of(elem_of_words<DT>(sm.walk.t, lane), elem_of_words<DT>(sm.walk.d, lane),
                                          rmode, ot, od, P.sc)
                                : 0.f;
      float a = 0.f, al = 0.f;
#pragma unroll
      for (int l = 0; l < NE; ++l) {
        a += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), l));
        al = lane == l ? a : al;
      }
      const double wbase = sm.dbc[3];
      const uint64_t pass = __ballot(m > 0.f && prefix + (wbase + (double)al) > tau);
      const uint64_t posm = __ballot(m > 0.f);
      const int e = pass ? __builtin_ctzll(pass) : (posm ? 63 - __builtin_clzll(posm) : -1);
      pos = e < 0 ? -1 : walker * NE + e;
    }
    if (lane == 0) {
      if (state == 0) state = wait_at_least(&rec->state, 1, P.fault);
      if (state == 1) P.out_tokens[(int64_t)b * K1 + j] = pos < 0 ? -1 : c * Fmt<DT>::TILE + pos;
    }
  }
}

// Draw workgroup (b, c), dispatched after every streaming workgroup.  It
// learns the drawing row j of sequence b from the group records as soon as it
// is decided: the first rejected draft (all earlier ones accepted), or row k
// once all k drafts are accepted; with more than 63 drafts it waits for the
// sequence's assembly instead.  For a residual (j < k) it publishes tile c's
// total mass of max(0, p_j - q_j), waits for the row's other tiles and finds
// the crossing tile of tau = u * R over the totals in tile order; for the
// bonus (j == k) the tile masses of p_k come from row k's tile records
// (sum times 2^(max * sc - ot)), so no tile is read before the crossing is
// known.  The workgroup that holds the crossing tile draws the first
// positive-mass element whose cumulative mass exceeds tau (the tile's last
// positive-mass element should rounding leave none), written once the
// assembly has found no data error.  A residual with no mass left (only through rounding) is
// replaced by p_j in a second round.  Within a tile, cumulative masses are the
// fixed-order fp64 scan of fp32 per-thread sums (for a residual the same
// arithmetic as its tile totals; a bonus tile's total from the statistics
// agrees with its elements' sum to rounding, and the fallback above covers a
// crossing that rounding moves past the tile's end).  A sequence's draw workgroups are consecutive, so each waits
// only for workgroups dispatched with it or before it.  The last one to finish
// clears the sequence's state.
template <int DT, bool HI>
__device__ __forceinline__ void draw_tile(const Params &P, int b, int c, Smem &sm) {
  constexpr int W = Fmt<DT>::W;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT, k = P.k, K1 = k + 1;
  SeqRec *rec = (SeqRec *)((char *)P.srec + (int64_t)b * SREC_STRIDE);
  const GroupRec *grs = P.grec + (int64_t)b * K1;
  if (wid == 0) {
    // the residual's and the bonus's uniforms, read before the drawing row is known
    const float ures = P.uniforms[(int64_t)b * (k + 2) + k], ubon = P.uniforms[(int64_t)b * (k + 2) + k + 1];
    int j = -1;
    uint64_t ow = 0;                   // lane i: group i's offsets word
    if (K1 <= 64) {
      // lane i watches group i's (accept, ready) word and its offsets word
      const uint64_t *word = (const uint64_t *)&grs[lane < K1 ? lane : 0].accept;
      const uint64_t *oword = (const uint64_t *)&grs[lane < K1 ? lane : 0].ot;
      uint64_t w = lane < K1 ? ld_dev(word) : 0ull;
      ow = lane < K1 ? ld_dev(oword) : 0ull;
      const uint64_t all = K1 == 64 ? ~0ull : (1ull << K1) - 1;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        const uint64_t rdy = __ballot(lane < K1 && (w >> 32) != 0 && ow != 0) & all;
        const uint64_t rej = __ballot(lane < k && (w >> 32) != 0 && (uint32_t)w == 0u);
        const uint64_t nr = all & ~rdy;
        const int fz = nr ? __builtin_ctzll(nr) : K1;              // first group not yet in
        const uint64_t below = fz >= 64 ? ~0ull : (1ull << fz) - 1;
        if (rej & below) { j = __builtin_ctzll(rej & below); break; }
        if (fz == K1) { j = k; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
          if (lane == 0) atomicOr(P.fault, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
        if (lane < K1 && (w >> 32) == 0) w = ld_dev(word);
        if (lane < K1 && ow == 0) ow = ld_dev(oword);
      }
      if (j >= 0) ow = ((uint64_t)readlane((uint32_t)(ow >> 32), j) << 32) | readlane((uint32_t)ow, j);
    } else if (lane == 0) {
      const int v = wait_at_least(&rec->state, 1, P.fault);
      if (v == 1 || v == 2) j = ld_dev(&rec->j);
      if (j < 0 || j > k) { if (v > 0) atomicOr(P.fault, 2); j = -1; }
      j = v == 1 ? j : -1;
      if (j >= 0) ow = ld_dev((const uint64_t *)&grs[j].ot);
    }
    if (lane == 0) {
      sm.bc[3] = j;
      if (j >= 0) {
        sm.f[2][0] = __uint_as_float(~(uint32_t)ow);
        sm.f[2][1] = __uint_as_float(~(uint32_t)(ow >> 32));
        sm.dbc[2] = (double)(j < k ? ures : ubon);
      }
    }
  }
  __syncthreads();
  const int j = sm.bc[3];
  uint64_t *tot = P.dtot + (int64_t)b * nT * 2;
  if (j == k) {
    // bonus draw: the crossing tile straight from row k's streaming
    // statistics, which its merge leaves for the draw.  Tile t's mass under
    // p = exp2(x * sc - ot) is s_t * 2^(m_t * sc - ot), s_t its sum of
    // exp2((x - m_t) * sc) (lane t, in tile order); only the workgroup that
    // holds the crossing reads its elements
    const float ot = sm.f[2][0];
    if (wid == 0) {
      const uint64_t *rk = (const uint64_t *)(P.recs + (int64_t)(b * K1 + k) * nT) + lane * 8;
      const bool own = lane < nT;
      constexpr uint64_t cpl = Uncounted<DT, false, HI> ? ~0ull : 0ull;   // complemented records
      const uint64_t w0 = own ? ld_dev(rk) ^ cpl : 0ull, w1 = own ? ld_dev(rk + 1) ^ cpl : 0ull;
      const float mt = __uint_as_float((uint32_t)w0);
      const double tm = own && mt != NEG_INF
                            ? __builtin_bit_cast(double, w1) * exp2_split((double)mt * (double)P.sc - (double)ot)
                            : 0.0;
      const double cum = wave_scan_d(tm);
      const double tau = sm.dbc[2] * readlane_d(cum, 63);
      const uint64_t h = __ballot(own && cum > tau);
      const int cs = h ? __builtin_ctzll(h) : nT - 1;
      const double before = cs > 0 ? readlane_d(cum, cs - 1) : 0.0;
      if (lane == 0) { sm.bc[2] = cs; sm.dbc[0] = before; sm.dbc[1] = tau; }
    }
    __syncthreads();
    if (sm.bc[2] == c) {
      u32x4 rt[NSEG];
      load_tile<DT, true>(P.target + ((int64_t)b * K1 + k) * P.tstride * Fmt<DT>::E, c, P.V, P.t_vec, rt);
      float a = 0.f;
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int w = 0; w < W; ++w) a += draw_mass<DT>(rt[s], rt[s], w, false, ot, 0.f, P.sc);
      double base;
      block_scan_d((double)a, base, sm.d[0]);
      draw_crossing<DT>(P, b, c, j, rt, rt, false, ot, 0.f, a, base, rec, sm);
    }
  } else if (j >= 0) {
    const bool resid = true;           // j < k: the residual of pair row j
    const float ot = sm.f[2][0], od = sm.f[2][1];
    // (the high-occupancy build reads the uniform where it is used, one value
    // fewer held across the masses)
    const double u = HI ? 0.0 : sm.dbc[2];
    const char *trow = P.target + ((int64_t)b * K1 + j) * P.tstride * Fmt<DT>::E;
    const char *drow = resid ? P.draft + ((int64_t)b * k + j) * P.dstride * Fmt<DT>::E : nullptr;
    u32x4 rt[NSEG], rd[NSEG];
    load_tile<DT, true>(trow, c, P.V, P.t_vec, rt);
    if (resid) load_tile<DT, true>(drow, c, P.V, P.d_vec, rd);
    else
#pragma unroll
      for (int s = 0; s < NSEG; ++s) rd[s] = rt[s];
    bool rmode = resid;
    float mine = 0.f;                  // mass of this thread's elements, summed in order
    double base = 0.0;                 // mass of the tile's elements before them
#pragma unroll 1
    for (int round = 0; round < 2; ++round) {
      // the thread's sum, its scan over the tile, and the tile total.  The
      // offsets and data pass through an empty asm so that the compiler
      // unpacks and computes the masses here, element by element, instead of
      // hoisting them out of the loop and keeping them live
      float o1 = ot, o2 = od;
      asm volatile("" : "+v"(o1), "+v"(o2));
#pragma unroll
      for (int s = 0; s < NSEG; ++s) asm volatile("" : "+v"(rt[s]), "+v"(rd[s]));
      float a = 0.f;
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int w = 0; w < W; ++w) a += draw_mass<DT>(rt[s], rd[s], w, rmode, o1, o2, P.sc);
      mine = a;
      const double t = block_scan_d((double)a, base, sm.d[0]);
      if (tid == 0) st_dev(tot + 2 * c + round, tot_word(t));
      // the crossing tile, from the totals in tile order (wave 0, lane l
      // polling tile l's slot until every tile has published)
      if (wid == 0) {
        uint64_t tw = lane < nT ? ld_dev(tot + 2 * lane + round) : ~0ull;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__ballot(tw == 0)) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
            if (lane == 0) atomicOr(P.fault, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
          if (tw == 0) tw = ld_dev(tot + 2 * lane + round);
        }
        const double cum = wave_scan_d(lane < nT ? tot_value(tw) : 0.0);
        const double R = readlane_d(cum, 63);
        const double tau = (HI ? sm.dbc[2] : u) * R;
        const uint64_t h = __ballot(lane < nT && cum > tau);
        const int cs = h ? __builtin_ctzll(h) : nT - 1;
        const double before = cs > 0 ? readlane_d(cum, cs - 1) : 0.0;
        if (lane == 0) { sm.bc[2] = cs; sm.bc[4] = (rmode && !(R > 0.0)) ? 1 : 0; sm.dbc[0] = before; sm.dbc[1] = tau; }
      }
      __syncthreads();
      if (!sm.bc[4]) break;
      rmode = false;                   // no residual mass left: draw from p_j
    }
    // (fp32: j read again from LDS, not held in registers across the rounds,
    // which keeps this build within 64 registers without spilling)
    const int jc = DT == SV_F32 ? *(volatile int32_t *)&sm.bc[3] : j;
    if (sm.bc[2] == c) draw_crossing<DT>(P, b, c, jc, rt, rd, rmode, ot, od, mine, base, rec, sm);
  }
  // every draw workgroup of the sequence reports; the last clears its state
  const int old = count_done(P.ddone + (int64_t)b * CTR, &sm.bc[7]);
  if (old != nT - 1) {
    if ((old < 0 || old >= nT) && tid == 0) atomicOr(P.fault, 2);
    return;
  }
  // (the assembly has read the group records once it has set its state)
  if (tid == 0) wait_at_least(&rec->state, 1, P.fault);
  __syncthreads();
  for (int q = tid; q < 2 * nT; q += TPB) st_dev(tot + q, (uint64_t)0);
  zero_recs(rec, 1);
  zero_recs(P.grec + (int64_t)b * K1, K1);
  {
    uint64_t *rk = (uint64_t *)(P.recs + (int64_t)(b * K1 + k) * nT);   // row k's words 0-1, left by its merge
    for (int q = tid; q < 2 * nT; q += TPB) st_dev(rk + (q >> 1) * 8 + (q & 1), (uint64_t)0);
  }
  if (tid == 0) st_dev(P.ddone + (int64_t)b * CTR, 0);
}

template <int DT, bool GREEDY, bool HI>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(kWaves<DT, GREEDY, HI>, 8))) void sv_verify(Params P) {
  __shared__ Smem sm;
  constexpr int W = Fmt<DT>::W, TILE = Fmt<DT>::TILE;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int V = P.V;
  if (!GREEDY && (int)blockIdx.x >= P.items) {           // draw workgroups come last
    const int d = blockIdx.x - P.items;
    int b = d / P.nT;
    if constexpr (HI) b = __builtin_amdgcn_readfirstlane(b);   // kept in a scalar register
    draw_tile<DT, HI>(P, b, d - b * P.nT, sm);
    return;
  }
  const int item = P.xcd_runs ? xcd_item(blockIdx.x, P.items) : (int)blockIdx.x;
  const Geo G = geo<DT, GREEDY>(P, item);
  const int c = G.c;
  const bool pair = G.pair;
  // the drafted token of a pair group (used only by the group's merge)
  const int32_t xtok = pair ? P.tokens[(int64_t)G.b * P.k + G.i] : -1;

  u32x4 rt[NSEG], rd[NSEG];
  load_tile<DT, false, NSEG, kStreamNT<DT>>(G.trow, c, V, P.t_vec, rt);
  if (pair) load_tile<DT, false, NSEG, kStreamNT<DT>>(G.drow, c, V, P.d_vec, rd);
  if (tid == 0) sm.bc[0] = 0;                          // candidate count

  // wave maxima, exp sums and flags: the draft part first (its elements are
  // not needed afterwards), then the target part, each unpacked once
  float wm_t, wm_d = NEG_INF;
  double ws_t = 0.0, ws_d = 0.0;
  int wf_t = 0, wf_d = 0;
  if (pair) {
    Elems<DT> ed;
    unpack_all<DT>(rd, ed);
    float md = vmax_of<DT>(ed, 0);
#pragma unroll
    for (int s = 1; s < NSEG; ++s) md = fmax_nan(md, vmax_of<DT>(ed, s));
    wave_stats<DT>(ed, md, P.sc, wm_d, ws_d, wf_d);
  }
  Elems<DT> et;
  unpack_all<DT>(rt, et);
  float vmt[NSEG];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) vmt[s] = vmax_of<DT>(et, s);
  float mt = vmt[0];
#pragma unroll
  for (int s = 1; s < NSEG; ++s) mt = fmax_nan(mt, vmt[s]);
  if (!GREEDY) {
    wave_stats<DT>(et, mt, P.sc, wm_t, ws_t, wf_t);
  } else {
    wm_t = wave_max_f(mt);
    wf_t = __ballot(has_nan_of<DT>(et)) ? SV_STATUS_NAN : 0;   // no exp sums here: test every element
  }

  // the wave's two largest lane maxima
  const bool has_elem = (int64_t)c * TILE + (int64_t)tid * W < V;
  const uint32_t tkey = has_elem ? ordered_key(mt) : 0u;
  uint32_t k1, k2;
  wave_top2(tkey, k1, k2);
  if (lane == 0) {
    sm.w8[2 * wid] = k1; sm.w8[2 * wid + 1] = k2;
    sm.f[0][wid] = wm_t; sm.f[1][wid] = wm_d; sm.i[0][wid] = wf_t; sm.i[1][wid] = wf_d;
    sm.d[0][wid] = ws_t; sm.d[1][wid] = ws_d;
  }
  __syncthreads();
  // the candidate threshold: the smallest nonzero of the tile's 8 lane maxima
  // (8 distinct lanes hold an element at or above it); 0 in an empty tile
  uint32_t kthr = 0xffffffffu;
#pragma unroll
  for (int q = 0; q < LIST; ++q) { const uint32_t v = sm.w8[q]; if (v && v < kthr) kthr = v; }
  if (kthr == 0xffffffffu) kthr = 0u;

  // candidates: elements at or above the threshold.  Every vector whose
  // maximum reaches it is staged raw in LDS with its tile position (one LDS
  // slot reservation per wave and vector, no per-element work); wave 0 takes
  // the candidates out of the staged vectors and forms the ordered keys of
  // those it publishes
  const float thr = key_value(kthr);
  const int lim = V - c * TILE;                          // tile positions < lim exist
  {
    const bool act = has_elem && tkey >= kthr;           // lanes that may hold candidates
    // (the high-occupancy bf16 sampling build, at 64 registers, packs a
    // staged vector again from its unpacked elements, so that the packed tile
    // is not held live across the statistics)
    constexpr bool REPACK = DT == SV_BF16 && HI && !GREEDY;
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      if (act && vmt[s] >= thr) {
        const int slot = atomicAdd(&sm.bc[0], 1);
        if (slot < STAGE_V) {
          sm.st.v[slot] = REPACK ? repack<DT>(et, s) : rt[s];
          sm.st.pos[slot] = tpos<DT>(s, 0);
        }
      }
    }
  }
  // wave 0 publishes the record and the candidates (one store for all of
  // them), so the other waves of a tile that does not merge are done here
  constexpr bool UNC = Uncounted<DT, GREEDY, HI>;
  const bool last = c == P.nT - 1;
  __syncthreads();
  if (wid != 0 && !last) return;

  // the tile record (wave 0: lanes 0-7 write one word each)
  if (wid == 0) {
    const TileStats ts = tile_stats<GREEDY>(sm, P.sc);
    // the candidates of the staged vectors (lane q: vector q), element by
    // element, packed by ballot as value bits and tile position
    const int nv = sm.bc[0];
    const int nvs = nv < STAGE_V ? nv : STAGE_V;
    int nc = 0;
    for (int q0 = 0; q0 < nvs; q0 += 64) {
      const int q = q0 + lane;
      const bool have = q < nvs;
      const u32x4 v = have ? sm.st.v[q] : u32x4{0u, 0u, 0u, 0u};
      const int p0 = have ? sm.st.pos[q] : 0;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float e = unpack<DT>(v, w);
        const bool hit = have && p0 + w < lim && e >= thr;
        const uint64_t m = __ballot(hit);
        if (hit) {
          const int at = nc + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (at < STAGE) sm.st.ck[at] = raw_cand(e, p0 + w);
        }
        nc += (int)__builtin_popcountll(m);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // more vectors than the stage holds, or more candidates: the merge
    // rescans.  More candidates than slots, all of them staged: the tile
    // publishes its own 32 largest (by key, ranked by counting) and a
    // threshold of 0.  Its other elements each lie below 32 published ones,
    // so none can be among the row's 32 largest and the merge never rescans
    // the tile
    const bool ovf = nv > STAGE_V || nc > STAGE;
    const bool own32 = !ovf && nc > SLOTS;
    // the staged candidates' keys: every one of them to rank the tile's own
    // 32 largest, else the first SLOTS
    const int nk = own32 ? nc : (nc < SLOTS ? nc : SLOTS);
    for (int q = lane; q < nk; q += 64) sm.st.ck[q] = key_of_raw(sm.st.ck[q], c * TILE);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the slots first, then the record, whose words go out complemented (a
    // NaN maximum or sum and an all-ones key canonical, so no word is 0 once
    // written): the merge reads a word again until it is nonzero, and takes
    // the record's count of slots in use, with no store wait and no counter
    // between the tile and its merge
    const int npub = own32 ? SLOTS : (nc < SLOTS ? nc : SLOTS);
    if (!own32) {
      if (lane < npub) st_dev(P.cand + (int64_t)item * SLOTS + lane, sm.st.ck[lane]);
    } else {
      for (int q = lane; q < nc; q += 64) {
        const uint64_t kq = sm.st.ck[q];
        int rank = 0;
        for (int jj = 0; jj < nc; ++jj) rank += sm.st.ck[jj] > kq;
        if (rank < SLOTS) st_dev(P.cand + (int64_t)item * SLOTS + rank, kq);
      }
    }
    if (lane < 8) {
      auto canon_k = [](uint32_t v) { return UNC && v == 0xffffffffu ? 0xfffffffeu : v; };
      uint64_t word;
      if (lane < 3) word = stat_word<UNC>(ts, lane);
      else if (lane == 3)
        word = ((uint64_t)(own32 ? 0u : kthr) << 32) | (uint32_t)(ts.f_t | (ts.f_d << 8)) | ((uint32_t)npub << 16) |
               (ovf ? 1u << 24 : 0u);
      else word = ((uint64_t)canon_k(sm.w8[2 * (lane - 4) + 1]) << 32) | canon_k(sm.w8[2 * (lane - 4)]);
      st_dev((uint64_t *)(P.recs + item) + lane, UNC ? ~word : word);
    }
    // counted: the stores complete before the count
    if (!UNC) {
      stores_done();
      if (!last && lane == 0) add_dev_noret(P.garrive + (int64_t)G.g * CTR, 1);
    }
  }
  if (!last) return;                                     // not the group's last tile: done
  if (!UNC) {
    // the group's last tile waits for the others' count before it merges
    if (tid == 0) {
      const int v = wait_at_least(P.garrive + (int64_t)G.g * CTR, P.nT - 1, P.fault);
      if (v > P.nT - 1) atomicOr(P.fault, 2);                        // workspace not zero-filled
      st_dev(P.garrive + (int64_t)G.g * CTR, 0);
    }
    __syncthreads();
  }
  group_finish<DT, GREEDY, HI>(P, G, xtok, sm);
}

// ---------------------------------------------------------------- host side
using sv_host::Layout;
using sv_host::layout_for;
using sv_host::shape_ok;
using sv_host::table_layout;
using sv_host::table_variant;
using sv_host::tile_of;
static_assert(sizeof(TileRec) == sv_host::TILE_REC_BYTES && sizeof(GroupRec) == sv_host::GROUP_REC_BYTES &&
                  SREC_STRIDE == (int)sv_host::SEQ_REC_BYTES && SLOTS == sv_host::SLOTS && CTR == sv_host::CTR &&
                  MAX_TILES == sv_host::MAX_TILES && Fmt<SV_BF16>::TILE == 8192 && Fmt<SV_F32>::TILE == 4096,
              "host layout constants");

template <int DT>
hipError_t launch(const Params &P, bool greedy, bool hi, hipStream_t stream) {
  // streaming workgroups, then (sampling) one draw workgroup per (sequence, tile);
  // fp32 has one build
  const unsigned grid = (unsigned)P.items + (greedy ? 0u : (unsigned)P.B * (unsigned)P.nT);
  if constexpr (DT == SV_BF16) {
    if (hi) {
      if (greedy) hipLaunchKernelGGL((sv_verify<DT, true, true>), dim3(grid), dim3(TPB), 0, stream, P);
      else hipLaunchKernelGGL((sv_verify<DT, false, true>), dim3(grid), dim3(TPB), 0, stream, P);
      return hipGetLastError();
    }
  }
  if (greedy) hipLaunchKernelGGL((sv_verify<DT, true, false>), dim3(grid), dim3(TPB), 0, stream, P);
  else hipLaunchKernelGGL((sv_verify<DT, false, false>), dim3(grid), dim3(TPB), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

extern "C" int spec_verify_layout_choice(const sv_shape_t *s) {
  if (!s || !shape_ok(s) || !(s->temperature >= 0.f) || s->temperature == __builtin_inff()) return 0;
  return table_layout(s);
}

extern "C" int spec_verify_variant_choice(const sv_shape_t *s) {
  if (!s || !shape_ok(s) || !(s->temperature >= 0.f) || s->temperature == __builtin_inff()) return 0;
  return table_variant(s);
}

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
    case SV_ERR_SCRATCH:
      return "spec_verify_noalloc: the shape needs more workspace than its static scratch (SV_NOALLOC_MAX_BYTES, "
             "8 MiB); call spec_verify with a workspace instead";
    default: return "unknown error code";
  }
}

// ---------------------------------------------------------------- no-allocation entry
// The workspace of spec_verify_noalloc: one copy of this array per GPU, held
// until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[SV_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SV_OK;
}

// Zero n16 16-byte words with vector stores.
__global__ __launch_bounds__(256) void sv_zero_fill(u32x4 *p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) p[i] = z;
}

// Both entry points: validation, then (noalloc) the scratch clear, then the launch.
int verify_impl(const sv_shape_t *shape, const void *target_logits, const void *draft_logits,
                const int32_t *draft_tokens, const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                float *topk_val, int32_t *topk_idx, const sv_aux_t *aux, void *workspace, size_t workspace_bytes,
                void *stream, bool noalloc) {
  bool nothing = false;
  const int rc0 = sv_host::check_args(shape, target_logits, draft_logits, draft_tokens, uniforms, accepted_len,
                                      out_tokens, topk_val, topk_idx, aux, &nothing);
  if (rc0 != SV_OK || nothing) return rc0;
  const sv_shape_t s = *shape;
  const int64_t ts = s.target_row_stride ? s.target_row_stride : s.V;
  const int64_t ds = s.draft_row_stride ? s.draft_row_stride : s.V;
  const int64_t nT = ((int64_t)s.V + tile_of(s.dtype) - 1) / tile_of(s.dtype);
  const int64_t items = (int64_t)s.B * (s.k + 1) * nT;
  const bool greedy = s.temperature == 0.f;
  const int req_layout = aux ? aux->item_layout : SV_LAYOUT_AUTO;
  const int req_variant = aux ? aux->variant : SV_VARIANT_AUTO;
  const Layout L = layout_for(s.B, s.k, s.V, s.dtype);
  if (noalloc) {
    if (L.total > (size_t)SV_NOALLOC_MAX_BYTES) return SV_ERR_SCRATCH;
    const int rc = scratch_address(&workspace);
    if (rc != SV_OK) return rc;
    workspace_bytes = SV_NOALLOC_MAX_BYTES;
    // the array keeps the last call's contents: clear what this call uses
    const size_t n16 = L.total / 16;
    const unsigned g = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(sv_zero_fill, dim3(g), dim3(256), 0, (hipStream_t)stream, (u32x4 *)workspace, n16);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  }
  const int rc1 = sv_host::check_workspace(L, workspace, workspace_bytes);
  if (rc1 != SV_OK) return rc1;

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
  P.ddone = (int32_t *)(ws + L.ddone);
  P.recs = (TileRec *)(ws + L.recs);
  P.grec = (GroupRec *)(ws + L.grec);
  P.srec = (SeqRec *)(ws + L.srec);
  P.cand = (uint64_t *)(ws + L.cand);
  P.dtot = (uint64_t *)(ws + L.dtot);
  P.B = s.B;
  P.k = s.k;
  P.V = s.V;
  P.nT = (int32_t)nT;
  P.items = (int32_t)items;
  P.xcd_runs = (req_layout == SV_LAYOUT_AUTO ? table_layout(&s) : req_layout) == SV_LAYOUT_XCD_RUNS ? 1 : 0;
  P.T = greedy ? 0.f : s.temperature;
  P.scd = greedy ? 0.0 : 1.4426950408889634 / (double)s.temperature;
  P.sc = (float)P.scd;
  P.t_vec = (((uintptr_t)target_logits & 15) == 0 && ((ts * esz) & 15) == 0) ? 1 : 0;
  P.d_vec = (!greedy && s.k > 0 && ((uintptr_t)draft_logits & 15) == 0 && ((ds * esz) & 15) == 0) ? 1 : 0;

  const bool hi = (req_variant == SV_VARIANT_AUTO ? table_variant(&s) : req_variant) == SV_VARIANT_HIGH_OCC;
  const hipError_t e = s.dtype == SV_BF16 ? launch<SV_BF16>(P, greedy, hi, (hipStream_t)stream)
                                          : launch<SV_F32>(P, greedy, hi, (hipStream_t)stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" int spec_verify(const sv_shape_t *shape, const void *target_logits, const void *draft_logits,
                           const int32_t *draft_tokens, const float *uniforms, int32_t *accepted_len,
                           int32_t *out_tokens, float *topk_val, int32_t *topk_idx, const sv_aux_t *aux,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return verify_impl(shape, target_logits, draft_logits, draft_tokens, uniforms, accepted_len, out_tokens, topk_val,
                     topk_idx, aux, workspace, workspace_bytes, stream, false);
}

extern "C" int spec_verify_noalloc(const sv_shape_t *shape, const void *target_logits, const void *draft_logits,
                                   const int32_t *draft_tokens, const float *uniforms, int32_t *accepted_len,
                                   int32_t *out_tokens, float *topk_val, int32_t *topk_idx, const sv_aux_t *aux,
                                   void *stream) {
  return verify_impl(shape, target_logits, draft_logits, draft_tokens, uniforms, accepted_len, out_tokens, topk_val,
                     topk_idx, aux, nullptr, 0, stream, true);
}
