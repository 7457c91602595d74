// sv_device.h -- device helpers shared by the kernels of this library: launch
// constants, tile formats, DPP wave reductions and scans, device-scope loads,
// stores and bounded waits, and tile loads.  gfx950 (MI355X), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv_dev {

constexpr int TPB = 256;               // threads per workgroup (4 waves of 64)
constexpr int NWAVE = TPB / 64;
constexpr int NSEG = 4;                // 16-byte vectors per thread per row
constexpr float NEG_INF = -__builtin_inff();
constexpr uint64_t SPIN_TICKS = 20000000;          // bounded waits give up after 0.2 s (100 MHz clock)
constexpr int CTR = 64;                            // int32 per counter: each on its own 256 bytes, so
                                                   // polling one never contends with another

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The larger of a and b, NaN when either is (IEEE maximum).  gfx950 takes it
// in v_maximum3_f32 with no quieting of signalling-NaN inputs first, which the
// NaN-skipping fmaxf needs: about half the instructions per element.  The
// kernels find data NaNs from their exp sums and element tests, not from maxima.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// E: bytes per element; W: elements per 16-byte vector; TILE: elements per tile;
// LOW: key bits below the 16-bit bucket that no element of the format can vary
template <int DT> struct Fmt;
template <> struct Fmt<SV_BF16> {
  static constexpr int E = 2, W = 8, TILE = TPB * NSEG * 8, WAVES = 6;
  static constexpr uint32_t LOW = 0xffffu;   // low key bits of a bf16 value are all 0 or all 1
};
template <> struct Fmt<SV_F32> {
  static constexpr int E = 4, W = 4, TILE = TPB * NSEG * 4, WAVES = 7;
  static constexpr uint32_t LOW = 0u;
};

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
struct OpMaxI { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return (int)a > (int)b ? a : b; } };
struct OpMinI { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return (int)a < (int)b ? a : b; } };
struct OpOr { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
struct OpMaxF {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmax_nan(__uint_as_float(a), __uint_as_float(b)));
  }
};
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

__device__ __forceinline__ int wave_sum_i(int v) {
  v += (int)dpp<0x111, 0xf, 0xf>(0u, (uint32_t)v);
  v += (int)dpp<0x112, 0xf, 0xf>(0u, (uint32_t)v);
  v += (int)dpp<0x114, 0xf, 0xe>(0u, (uint32_t)v);
  v += (int)dpp<0x118, 0xf, 0xc>(0u, (uint32_t)v);
  v += (int)dpp<0x142, 0xa, 0xf>(0u, (uint32_t)v);
  v += (int)dpp<0x143, 0xc, 0xf>(0u, (uint32_t)v);
  return (int)readlane((uint32_t)v, 63);
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += __uint_as_float(dpp<0x111, 0xf, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<0x112, 0xf, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<0x114, 0xf, 0xe>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<0x118, 0xf, 0xc>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<0x142, 0xa, 0xf>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp<0x143, 0xc, 0xf>(0u, __float_as_uint(v)));
  return __uint_as_float(readlane(__float_as_uint(v), 63));
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
__device__ __forceinline__ void add_dev_noret(int32_t *p, int v) {
  (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's earlier memory accesses have completed (and keep the
// compiler from moving memory accesses across the wait).
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
// Bounded wait of one thread until *p >= target.  Returns the value seen;
// on timeout sets fault bit 1 and returns what it last saw.
__device__ __forceinline__ int wait_at_least(const int32_t *p, int target, int32_t *fault) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int v = ld_dev(p);
  while (v < target) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
      atomicOr(fault, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
    v = ld_dev(p);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return v;
}
// A published fp64 value that is its own flag: the complement of its bits,
// with -0 and NaN canonical, is never 0, the value of an empty slot.
__device__ __forceinline__ uint64_t tot_word(double t) {
  const double c = t == t ? t + 0.0 : __builtin_nan("");
  return ~__builtin_bit_cast(uint64_t, c);
}
__device__ __forceinline__ double tot_value(uint64_t w) { return __builtin_bit_cast(double, ~w); }

// Count this workgroup as done with the shared state it read; returns the
// count before it (the same value in every thread), passed through the LDS word
// slot.  Its stores need not complete first: the last one to count only clears
// state the others have read, and their reads are complete (their values were
// used before the barrier).
__device__ __forceinline__ int count_done(int32_t *ctr, int32_t *slot) {
  __syncthreads();
  if (threadIdx.x == 0) *slot = add_dev(ctr, 1);
  __syncthreads();
  const int old = *slot;
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

// tile-local position of element w of this thread's vector s when each thread
// owns NSEG consecutive vectors (the draw's order)
template <int DT> __device__ __forceinline__ int dpos(int s, int w) {
  return ((int)threadIdx.x * NSEG + s) * Fmt<DT>::W + w;
}

// Load one tile of a row into registers; entries past V read as -inf.
// Streaming (TM false): vector s of a thread sits at tpos (vectors interleaved
// over the threads).  Draw (TM true): vector s sits at dpos (each thread's
// vectors consecutive).  NT marks the loads nontemporal (the default for
// streaming, where each logit is read once; the draw's re-read measured
// faster with ordinary loads).  NS vectors per thread (a tile of TPB * NS * W
// entries; NSEG unless given).
template <int DT, bool TM = false, int NS = NSEG, bool NT = !TM>
__device__ __forceinline__ void load_tile(const char *row, int c, int V, bool vec, u32x4 (&r)[NS]) {
  static_assert(!TM || NS == NSEG, "the draw order is defined for NSEG vectors");
  constexpr int E = Fmt<DT>::E, W = Fmt<DT>::W;
  const int64_t c0 = (int64_t)c * (TPB * NS * W);
  if (vec && c0 + TPB * NS * W <= V) {
    // the whole tile lies in the row (the usual case): unconditional loads
    const char *base = row + (c0 + (TM ? dpos<DT>(0, 0) : tpos<DT>(0, 0))) * E;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 *a = (const u32x4 *)(base + (int64_t)(TM ? s * W : s * TPB * W) * E);
      r[s] = NT ? __builtin_nontemporal_load(a) : *a;
    }
    return;
  }
  // the row's last tile, or a row without 16-byte alignment.  First every
  // vector that lies in the row, with no wait between the loads: vectors past
  // V hold -inf (set before the loads, so that no lane's constant waits for
  // another lane's load).  Then, element by element, a vector that straddles V
  // (at most one per row and tile, none when V is a multiple of the vector
  // width) or every vector of an unaligned row.
  constexpr uint32_t NEG = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int64_t e0 = c0 + (TM ? dpos<DT>(s, 0) : tpos<DT>(s, 0));
    r[s] = u32x4{NEG, NEG, NEG, NEG};
    if (vec && e0 + W <= V) {
      if (NT) r[s] = __builtin_nontemporal_load((const u32x4 *)(row + e0 * E));
      else r[s] = *(const u32x4 *)(row + e0 * E);
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int64_t e0 = c0 + (TM ? dpos<DT>(s, 0) : tpos<DT>(s, 0));
    if (!(vec && e0 + W <= V) && e0 < V) {
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

// s * exp2((m - M) * sc) in fp64: a partial sum relative to m, rescaled to M
__device__ __forceinline__ double rescale(double s, float m, float M, float sc) {
  return m == NEG_INF ? 0.0 : s * (double)__builtin_amdgcn_exp2f((m - M) * sc);
}

// Exclusive prefix (fp64) of one value per thread over the workgroup, in
// thread order: excl receives the sum over the threads before this one; returns
// the total.  part: NWAVE doubles of LDS.  Fixed association: identical bits
// wherever it is evaluated.
__device__ __forceinline__ double block_scan_d(double x, double &excl, double *part) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const double inc = wave_scan_d(x);
  const double prev = wave_prev_d(inc);
  if (lane == 63) part[wid] = inc;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int w = 0; w < NWAVE; ++w) {
    if (w < wid) off += part[w];
    tot += part[w];
  }
  excl = off + prev;
  __syncthreads();
  return tot;
}

// Work item of workgroup bid in a launch of n items.  The chip deals
// workgroups to its 8 XCDs round-robin (bid mod 8), each XCD dispatching its
// share in order; items are laid out so that XCD x takes one contiguous run of
// them, in order.  The tiles of one row (or group) then sit on one XCD and are
// dispatched together (a row on a run boundary spans two XCDs), instead of
// being spread over all eight, whose progress differs.
__device__ __forceinline__ int xcd_item(int bid, int n) {
  const int x = bid & 7, q = bid >> 3, base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + q;
}

}  // namespace sv_dev
