// sv_kd.hip -- reward-weighted distillation of the drafter over the stored
// top-32 soft targets, for gfx950 (MI355X).
//
// The step (ReSpec notes, "4 . G2": the target logits the verification
// computes are kept, top-32 per position, as the soft target of an on-policy
// KD of the drafter with loss KL(softmax(log p) || q_theta); "5 . G3": the
// per-sample KD loss is weighted by w(r), the reward normalised within its
// group and clipped): per row n, the drafter's log-normaliser over the whole
// vocabulary, the KL from the softmax of the 32 stored target logits to the
// drafter distribution, the sample weight, the weighted loss over all rows,
// and optionally the gradient w * (q - pt) with respect to the drafter logits.
//
// One launch, one workgroup per (row, tile); a tile is 16 KB of the drafter
// row (8192 bf16 or 4096 fp32 entries), held in registers from its load to
// its gradient store, so the row is read once.  Each workgroup publishes its
// tile's max, sum of exps and flags as self-flagging words; wave 0 of every
// workgroup of the row polls all of them (lane = tile) and combines them in
// tile order into the row's log-normaliser, the same bits in each workgroup.
// The row's workgroups are consecutive and wait (bounded) only for one
// another.  Tile 0 computes the KL and the row's loss term, and clears the
// row's words once every tile has read them; the workgroup that publishes the
// last term sums all of them in row order.  A stored id's gradient entry is
// patched by the thread that wrote the entry's vector, after it.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_device.h"
#include "sv_kd.h"

namespace {

using namespace sv_dev;

constexpr int KSEG = NSEG;               // 16-byte vectors per thread: 16 KB tiles
constexpr int KMAX_TILES = 64;           // tiles per row: one polling lane each
constexpr int KTOP = 32;                 // stored entries per row
constexpr double LN2 = 0.6931471805599453;
constexpr double LOG2E = 1.4426950408889634;

template <int DT> constexpr int ktile() { return TPB * KSEG * Fmt<DT>::W; }

struct KParams {
  const char *z;                         // drafter logits
  int64_t zstride;                       // row stride, elements
  const float *tval;
  const int32_t *tidx, *row_sample;
  const float *rewards;
  float *kl, *weight;
  int32_t *status;
  double *loss;
  char *grad;                            // [N, V] or null
  int32_t N, V, nT, S, G;
  int32_t gdt;                           // gradient dtype
  int32_t z_vec, g_vec;                  // 16-byte aligned rows
  float w_max;
  int32_t *fault;                        // bit 1: a wait gave up; bit 2: workspace not zero-filled
  uint64_t *part;                        // [N][nT][3] tile max, tile sum, flags (self-flagging words)
  int32_t *rdone;                        // [N] tiles done, CTR int32 apart
  int32_t *ndone;                        // rows whose loss term is published
  double *term;                          // [N] loss term of the row
};

struct KSmem {
  double d[NWAVE];                       // tile statistics of the waves
  float f[NWAVE];
  int32_t i[NWAVE];
  double lse2;                           // the row's log2-normaliser (wave 0)
  int32_t zflags;                        // SV_KD_* bits of the drafter row (wave 0)
  double w;                              // the row's weight (wave 1)
  int32_t eflags;                        // SV_KD_* bits of the stored entries and sample id (wave 1)
  double pt[KTOP];                       // softmax of the stored entries (wave 1)
  double lpt[KTOP];                      // its logarithm
  int32_t px[KTOP];                      // token id of a used entry, else -1
  int32_t pcnt;                          // used entries whose id falls in this tile (wave 1)
  int32_t ppos[KTOP];                    // their positions in the tile, in entry order
  double ppt[KTOP];                      // and their pt
  double red[NWAVE];                     // final loss reduction
  int32_t slot;                          // counter values
};

// log2 of s > 0 to about 1e-7 absolute: the exponent exactly, the mantissa
// through the hardware log2.
__device__ __forceinline__ double kd_log2(double s) {
  int e;
  const double m = __builtin_frexp(s, &e);
  return (double)e + (double)__builtin_amdgcn_logf((float)m);
}

// The sample weight of row n: reward / group sum, clipped to [0, w_max]; 0 when
// the group sum is not positive.  Called by a whole wave; every workgroup of
// the row gets the same bits.  bad: the row's sample id is out of range.
__device__ __forceinline__ double row_weight(const KParams &P, int n, bool &bad) {
  const int lane = threadIdx.x & 63;
  const int s = P.row_sample[n];
  bad = s < 0 || s >= P.S;
  if (bad) return 0.0;
  const int g0 = (s / P.G) * P.G;
  double sum = 0.0;
  for (int l0 = 0; l0 < P.G; l0 += 64) {
    const double r = l0 + lane < P.G ? (double)P.rewards[g0 + l0 + lane] : 0.0;
    sum += wave_sum_d(r);
  }
  const double r = (double)P.rewards[s];
  double w = sum > 0.0 ? r / sum : 0.0;
  w = w > 0.0 ? w : 0.0;                 // negative and NaN weights count as 0
  return w < (double)P.w_max ? w : (double)P.w_max;
}

template <int DT> __device__ __forceinline__ uint32_t grad_bits(float g);
template <> __device__ __forceinline__ uint32_t grad_bits<SV_BF16>(float g) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)g);
}
template <> __device__ __forceinline__ uint32_t grad_bits<SV_F32>(float g) { return __float_as_uint(g); }

// Store the W gradient entries of one of the thread's vectors (columns col0 ..
// col0 + W - 1 of the row; entries at or past V are skipped).
template <int DT, int GT>
__device__ __forceinline__ void store_grad(char *grow, int64_t col0, int V, bool vec, const float (&g)[Fmt<DT>::W]) {
  constexpr int W = Fmt<DT>::W, GE = Fmt<GT>::E;
  if (vec && col0 + W <= V) {
    constexpr int WORDS = W * GE / 4;    // 32-bit words of the vector's gradient
    uint32_t u[WORDS];
#pragma unroll
    for (int q = 0; q < WORDS; ++q) {
      if constexpr (GT == SV_BF16) u[q] = grad_bits<SV_BF16>(g[2 * q]) | (grad_bits<SV_BF16>(g[2 * q + 1]) << 16);
      else u[q] = grad_bits<SV_F32>(g[q]);
    }
    if constexpr (WORDS == 2) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 v = {u[0], u[1]};
      __builtin_nontemporal_store(v, (u32x2 *)(grow + col0 * GE));
    } else {
#pragma unroll
      for (int h = 0; h < WORDS / 4; ++h) {
        u32x4 v = {u[4 * h], u[4 * h + 1], u[4 * h + 2], u[4 * h + 3]};
        __builtin_nontemporal_store(v, (u32x4 *)(grow + col0 * GE) + h);
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if (col0 + w >= V) break;
      if constexpr (GT == SV_BF16) ((uint16_t *)grow)[col0 + w] = (uint16_t)grad_bits<SV_BF16>(g[w]);
      else ((float *)grow)[col0 + w] = g[w];
    }
  }
}

// w * q over one tile: the thread's vectors, as stored at tpos.
template <int DT, int GT>
__device__ __forceinline__ void grad_tile(const KParams &P, const u32x4 (&r)[KSEG], int n, int c, bool zero,
                                          float hi, float corr, float wf) {
  constexpr int W = Fmt<DT>::W, TILE = ktile<DT>();
  char *grow = P.grad + (int64_t)n * P.V * Fmt<GT>::E;
  const float sc = (float)LOG2E;
#pragma unroll
  for (int s = 0; s < KSEG; ++s) {
    float g[W];
#pragma unroll
    for (int w = 0; w < W; ++w)
      g[w] = zero ? 0.f : wf * (__builtin_amdgcn_exp2f(fmaf(unpack<DT>(r[s], w), sc, -hi)) * corr);
    store_grad<DT, GT>(grow, (int64_t)c * TILE + tpos<DT>(s, 0), P.V, P.g_vec, g);
  }
}

template <int DT>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(6, 8))) void sv_kd_kernel(KParams P) {
  __shared__ KSmem sm;
  constexpr int W = Fmt<DT>::W, TILE = ktile<DT>();
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nT = P.nT;
  // (rows in launch order: dealing each XCD a contiguous run of rows, as the
  // verification kernel does, measured 1.7x slower here)
  const int n = blockIdx.x / nT, c = blockIdx.x - (blockIdx.x / nT) * nT;
  const char *row = P.z + (int64_t)n * P.zstride * Fmt<DT>::E;
  const float sc = (float)LOG2E;

  u32x4 r[KSEG];
  load_tile<DT, false, KSEG>(row, c, P.V, P.z_vec, r);

  // ---- tile statistics: wave max, exps relative to it (fp32 per thread and
  // wave, the rounding of the reference corrected in fp64), waves in fp64
  float m = NEG_INF;
#pragma unroll
  for (int s = 0; s < KSEG; ++s)
#pragma unroll
    for (int w = 0; w < W; ++w) m = fmaxf(m, unpack<DT>(r[s], w));
  const float wm = wave_max_f(m);
  // the data pass through an empty asm: each pass unpacks its elements again
  // instead of the compiler keeping all of them unpacked across passes
#pragma unroll
  for (int s = 0; s < KSEG; ++s) asm volatile("" : "+v"(r[s]));
  const float ref = wm == NEG_INF ? 0.f : wm;
  const float chi = ref * sc, clo = fmaf(ref, sc, -chi);
  float st = 0.f;
#pragma unroll
  for (int s = 0; s < KSEG; ++s)
#pragma unroll
    for (int w = 0; w < W; ++w) st += __builtin_amdgcn_exp2f(fmaf(unpack<DT>(r[s], w), sc, -chi));
  int fl = 0;
  if (__ballot(!(st == st))) {
    bool nan = false;
#pragma unroll
    for (int s = 0; s < KSEG; ++s)
#pragma unroll
      for (int w = 0; w < W; ++w) { const float x = unpack<DT>(r[s], w); nan |= !(x == x); }
    fl = __ballot(nan) ? SV_KD_NAN : SV_KD_POSINF;
  }
  const double ws = (double)wave_sum_f(st) * (1.0 - (double)clo * LN2);
  if (lane == 0) { sm.f[wid] = wm; sm.d[wid] = ws; sm.i[wid] = fl; }
  __syncthreads();
  uint64_t *part = P.part + (int64_t)n * nT * 3;
  if (tid == 0) {
    float M = sm.f[0];
    int F = sm.i[0];
    for (int w = 1; w < NWAVE; ++w) { M = fmaxf(M, sm.f[w]); F |= sm.i[w]; }
    double S = 0.0;
    for (int w = 0; w < NWAVE; ++w) S += rescale(sm.d[w], sm.f[w], M, sc);
    st_dev(part + 3 * c + 0, tot_word((double)M));
    st_dev(part + 3 * c + 1, tot_word(S));
    st_dev(part + 3 * c + 2, tot_word((double)F));
  }

  if (wid == 0) {
    // ---- the row's log2-normaliser from every tile's words, in tile order
    uint64_t a0 = ~0ull, a1 = ~0ull, a2 = ~0ull;
    if (lane < nT) { a0 = ld_dev(part + 3 * lane); a1 = ld_dev(part + 3 * lane + 1); a2 = ld_dev(part + 3 * lane + 2); }
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__ballot(a0 == 0 || a1 == 0 || a2 == 0)) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
        if (lane == 0) atomicOr(P.fault, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
      if (a0 == 0) a0 = ld_dev(part + 3 * lane);
      if (a1 == 0) a1 = ld_dev(part + 3 * lane + 1);
      if (a2 == 0) a2 = ld_dev(part + 3 * lane + 2);
    }
    // this workgroup has read the row's words (their values are in hand)
    if (lane == 0) add_dev_noret(P.rdone + (int64_t)n * CTR, 1);
    const float mc = lane < nT ? (float)tot_value(a0) : NEG_INF;
    const float M = wave_max_f(mc);
    const double S = wave_sum_d(lane < nT ? rescale(tot_value(a1), mc, M, sc) : 0.0);
    int F = wave_or(lane < nT ? (int)tot_value(a2) : 0);
    F = (F & SV_KD_NAN) ? SV_KD_NAN : F;
    if (!F && M == NEG_INF) F = SV_KD_EMPTY;
    if (lane == 0) {
      sm.lse2 = (double)M * LOG2E + kd_log2(S);
      sm.zflags = F;
    }
  } else if (wid == 1) {
    // ---- the stored entries' softmax (fp64) and the row's weight
    bool badw;
    const double w = row_weight(P, n, badw);
    const float v = lane < KTOP ? P.tval[(int64_t)n * KTOP + lane] : NEG_INF;
    const int x = lane < KTOP ? P.tidx[(int64_t)n * KTOP + lane] : -1;
    const bool pad = lane >= KTOP || v == NEG_INF || x == -1;
    int F = 0;
    if (!pad && (x < 0 || x >= P.V)) F |= SV_KD_BAD_INDEX;
    if (lane < KTOP && !(v == v)) F |= SV_KD_NAN;
    if (lane < KTOP && v == __builtin_inff()) F |= SV_KD_POSINF;
    // an in-range id that an earlier non-padding entry already names: the
    // stored entries are then no distribution over tokens
    {
      const int mine = pad ? -1 : x, xs = (!pad && x >= 0 && x < P.V) ? x : -1;
      bool dup = false;
      for (int e = 0; e < KTOP; ++e) dup |= e < lane && xs >= 0 && __builtin_amdgcn_readlane(mine, e) == xs;
      if (dup) F |= SV_KD_DUP_INDEX;
    }
    F = wave_or(F) | (badw ? SV_KD_BAD_INDEX : 0);
    const bool use = !pad && !F;
    const float Mv = wave_max_f(use ? v : NEG_INF);
    if (!F && Mv == NEG_INF) F = SV_KD_EMPTY;
    const double a = use ? (double)v - (double)Mv : 0.0;
    const double e = use ? exp(a) : 0.0;
    const double Sv = wave_sum_d(e);
    if (lane < KTOP) {
      sm.pt[lane] = use ? e / Sv : 0.0;
      sm.lpt[lane] = use ? a - log(Sv) : 0.0;
      sm.px[lane] = use ? x : -1;
    }
    // the entries whose id falls in this tile, in entry order
    const bool here = use && x >= c * TILE && x < c * TILE + TILE;
    const uint64_t hm = __ballot(here);
    if (here) {
      const int q = __popcll(hm & ((1ull << lane) - 1));
      sm.ppos[q] = x - c * TILE;
      sm.ppt[q] = e / Sv;
    }
    if (lane == 0) { sm.w = w; sm.eflags = F; sm.pcnt = __popcll(hm); }
  }
  __syncthreads();
  const int F = sm.zflags | sm.eflags;
  const double lse2 = sm.lse2, w = sm.w;

  // ---- tile 0: the KL and the row's outputs
  bool last_row = false;
  if (c == 0 && wid == 0) {
    const int x = lane < KTOP ? sm.px[lane] : -1;
    double t = 0.0;
    if (!F && x >= 0 && sm.pt[lane] > 0.0) {
      const double zx = (double)load_elem<DT>(row, x);
      t = sm.pt[lane] * (sm.lpt[lane] - (zx - lse2 * LN2));
    }
    const double kl = wave_sum_d(t);
    if (lane == 0) {
      int st = F;
      if (ld_dev(P.fault)) st |= SV_KD_SYNC_TIMEOUT;
      P.kl[n] = st ? __builtin_nanf("") : (float)kl;
      if (P.weight) P.weight[n] = (float)w;
      if (P.status) P.status[n] = st;
      st_dev(P.term + n, (!st && w > 0.0) ? w * kl : 0.0);
      stores_done();
      last_row = add_dev(P.ndone, 1) == P.N - 1;
    }
    last_row = __ballot(last_row) != 0;
  }

  // ---- the gradient of this tile: w * q everywhere, then w * (q - pt) at the
  // stored ids that fall in it.  A patch is written by the thread that wrote
  // the entry's vector, after it in program order, so it lands last without a
  // wait for the tile's stores (a row's stored ids are distinct: a repeat is a
  // data error, so no two patches of a row meet).
  if (P.grad) {
    const float hi = (float)lse2, lo = (float)(lse2 - (double)hi);
    const float corr = 1.f - lo * (float)LN2;
    const float wf = (float)w;
#pragma unroll
    for (int s = 0; s < KSEG; ++s) asm volatile("" : "+v"(r[s]));
    if (P.gdt == SV_BF16) grad_tile<DT, SV_BF16>(P, r, n, c, F != 0, hi, corr, wf);
    else grad_tile<DT, SV_F32>(P, r, n, c, F != 0, hi, corr, wf);
    const int npatch = F ? 0 : sm.pcnt;
    for (int e = 0; e < npatch; ++e) {
      const int p = sm.ppos[e];
      if ((p / W) % TPB == tid) {
        const int64_t x = (int64_t)c * TILE + p;
        const float zx = load_elem<DT>(row, x);
        const float q = __builtin_amdgcn_exp2f(fmaf(zx, sc, -hi)) * corr;
        const float g = (float)((double)wf * ((double)q - sm.ppt[e]));
        char *grow = P.grad + (int64_t)n * P.V * (P.gdt == SV_BF16 ? 2 : 4);
        if (P.gdt == SV_BF16) ((uint16_t *)grow)[x] = (uint16_t)grad_bits<SV_BF16>(g);
        else ((float *)grow)[x] = g;
      }
    }
  }

  // ---- tile 0 clears the row's words once every tile has read them (the
  // others report right after reading, long before tile 0 gets here); the
  // last row sums the loss
  if (c != 0) return;
  if (tid == 0) {
    sm.slot = last_row ? 1 : 0;
    const int v = wait_at_least(P.rdone + (int64_t)n * CTR, nT, P.fault);
    if (v > nT) atomicOr(P.fault, 2);                  // workspace not zero-filled
  }
  __syncthreads();
  for (int q = tid; q < 3 * nT; q += TPB) st_dev(part + q, (uint64_t)0);
  if (tid == 0) st_dev(P.rdone + (int64_t)n * CTR, 0);
  if (!sm.slot) return;
  // every row's term is published: sum them in row order (a fixed chunk per
  // thread, then the waves in order), then clear them
  const int N = P.N, ch = (N + TPB - 1) / TPB;
  double acc = 0.0;
  for (int i = tid * ch; i < N && i < tid * ch + ch; ++i) acc += ld_dev(P.term + i);
  acc = wave_sum_d(acc);
  if (lane == 0) sm.red[wid] = acc;
  __syncthreads();
  if (tid == 0) {
    double L = 0.0;
    for (int q = 0; q < NWAVE; ++q) L += sm.red[q];
    P.loss[0] = L;
    st_dev(P.ndone, 0);
  }
  for (int i = tid; i < N; i += TPB) st_dev(P.term + i, 0.0);
}

struct KLayout {
  size_t fault, part, rdone, ndone, term, total;
};

size_t kalign(size_t x) { return (x + 255) & ~(size_t)255; }

int ktile_of(int dtype) { return dtype == SV_BF16 ? ktile<SV_BF16>() : ktile<SV_F32>(); }

bool kshape_ok(const sv_kd_shape_t *s) {
  if (s->N < 0 || s->V < 1) return false;
  if (s->dtype != SV_F32 && s->dtype != SV_BF16) return false;
  if (s->grad_dtype != SV_F32 && s->grad_dtype != SV_BF16) return false;
  if ((int64_t)s->V > (int64_t)KMAX_TILES * ktile_of(s->dtype)) return false;
  if (s->N > 0 && (s->S < 1 || s->group < 1 || s->S % s->group != 0)) return false;
  if (!(s->w_max > 0.f)) return false;
  return true;
}

KLayout klayout_for(int N, int V, int dtype) {
  const size_t nT = ((size_t)V + ktile_of(dtype) - 1) / ktile_of(dtype);
  KLayout L;
  size_t o = 0;
  L.fault = o; o = kalign(o + sizeof(int32_t));
  L.part = o;  o = kalign(o + (size_t)N * nT * 3 * sizeof(uint64_t));
  L.rdone = o; o = kalign(o + (size_t)N * CTR * sizeof(int32_t));
  L.ndone = o; o = kalign(o + CTR * sizeof(int32_t));
  L.term = o;  o = kalign(o + (size_t)N * sizeof(double));
  L.total = o;
  return L;
}

}  // namespace

extern "C" size_t sv_kd_workspace_bytes(const sv_kd_shape_t *s) {
  if (!s || !kshape_ok(s)) return 0;
  return klayout_for(s->N, s->V, s->dtype).total;
}

extern "C" int sv_kd(const sv_kd_shape_t *shape, const void *draft_logits, const float *topk_val,
                     const int32_t *topk_idx, const int32_t *row_sample, const float *rewards, float *kl,
                     float *weight, int32_t *status, double *loss, void *grad, void *workspace,
                     size_t workspace_bytes, void *stream) {
  if (!shape) return SV_ERR_NULL;
  const sv_kd_shape_t s = *shape;
  if (s.dtype != SV_F32 && s.dtype != SV_BF16) return SV_ERR_DTYPE;
  if (s.grad_dtype != SV_F32 && s.grad_dtype != SV_BF16) return SV_ERR_DTYPE;
  if (!kshape_ok(&s)) return SV_ERR_SHAPE;
  const int64_t zs = s.row_stride ? s.row_stride : s.V;
  if (zs < s.V) return SV_ERR_SHAPE;
  const int tile = ktile_of(s.dtype);
  const int64_t nT = ((int64_t)s.V + tile - 1) / tile;
  if ((int64_t)s.N * nT > 0x7fffffffLL) return SV_ERR_SHAPE;
  if (s.N == 0) return SV_OK;
  if (!draft_logits || !topk_val || !topk_idx || !row_sample || !rewards || !kl || !loss) return SV_ERR_NULL;
  const KLayout L = klayout_for(s.N, s.V, s.dtype);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;

  char *ws = (char *)workspace;
  const int esz = s.dtype == SV_BF16 ? 2 : 4, gsz = s.grad_dtype == SV_BF16 ? 2 : 4;
  KParams P;
  P.z = (const char *)draft_logits;
  P.zstride = zs;
  P.tval = topk_val;
  P.tidx = topk_idx;
  P.row_sample = row_sample;
  P.rewards = rewards;
  P.kl = kl;
  P.weight = weight;
  P.status = status;
  P.loss = loss;
  P.grad = (char *)grad;
  P.N = s.N;
  P.V = s.V;
  P.nT = (int32_t)nT;
  P.S = s.S;
  P.G = s.group;
  P.gdt = s.grad_dtype;
  P.z_vec = (((uintptr_t)draft_logits & 15) == 0 && ((zs * esz) & 15) == 0) ? 1 : 0;
  P.g_vec = (grad && ((uintptr_t)grad & 15) == 0 && (((int64_t)s.V * gsz) & 15) == 0) ? 1 : 0;
  P.w_max = s.w_max;
  P.fault = (int32_t *)(ws + L.fault);
  P.part = (uint64_t *)(ws + L.part);
  P.rdone = (int32_t *)(ws + L.rdone);
  P.ndone = (int32_t *)(ws + L.ndone);
  P.term = (double *)(ws + L.term);

  const dim3 grid((unsigned)((int64_t)s.N * nT)), block(TPB);
  if (s.dtype == SV_BF16) hipLaunchKernelGGL((sv_kd_kernel<SV_BF16>), grid, block, 0, (hipStream_t)stream, P);
  else hipLaunchKernelGGL((sv_kd_kernel<SV_F32>), grid, block, 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
