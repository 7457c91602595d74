// sv_host.h -- host-side argument checks, workspace layout and item-layout
// lookup of the verification library, in plain C++ with no HIP: the library
// includes it, and a CPU build with address and undefined-behaviour sanitizers
// drives it over valid and invalid shapes.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_dispatch.h"

namespace sv_host {

constexpr int TPB = 256;                 // threads per workgroup
constexpr int NSEG = 4;                  // 16-byte vectors per thread and row part of a tile
constexpr int MAX_TILES = 64;            // tiles per row: one merge lane each
constexpr int SLOTS = 32;                // candidate slots per tile
constexpr int CTR = 64;                  // int32 per counter (each on its own 256 bytes)
constexpr size_t TILE_REC_BYTES = 64;    // per (group, tile) record
constexpr size_t GROUP_REC_BYTES = 24;   // per group record
constexpr size_t SEQ_REC_BYTES = 256;    // per sequence record (its pollers share no line)

// elements per 16 KB tile
inline int tile_of(int dtype) { return dtype == SV_BF16 ? TPB * NSEG * 8 : TPB * NSEG * 4; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace sections, each 256-byte aligned, in this order; the fault word sits
// at offset 0 for every shape.
struct Layout {
  size_t fault, garrive, sarrive, ddone, recs, grec, srec, cand, dtot, total;
};

inline Layout layout_for(int B, int k, int V, int dtype) {
  const size_t groups = (size_t)B * (size_t)(k + 1);
  const size_t nT = ((size_t)V + tile_of(dtype) - 1) / tile_of(dtype);
  Layout L;
  size_t o = 0;
  L.fault = o;   o = align256(o + sizeof(int32_t));
  L.garrive = o; o = align256(o + groups * CTR * sizeof(int32_t));
  L.sarrive = o; o = align256(o + (size_t)B * CTR * sizeof(int32_t));
  L.ddone = o;   o = align256(o + (size_t)B * CTR * sizeof(int32_t));
  L.recs = o;    o = align256(o + groups * nT * TILE_REC_BYTES);
  L.grec = o;    o = align256(o + groups * GROUP_REC_BYTES);
  L.srec = o;    o = align256(o + (size_t)B * SEQ_REC_BYTES);
  L.cand = o;    o = align256(o + groups * nT * SLOTS * sizeof(uint64_t));
  L.dtot = o;    o = align256(o + (size_t)B * nT * 2 * sizeof(double));
  L.total = o;
  return L;
}

inline bool shape_ok(const sv_shape_t *s) {
  return s->B >= 0 && s->k >= 0 && s->V >= 1 && (s->dtype == SV_F32 || s->dtype == SV_BF16) &&
         (int64_t)s->V <= (int64_t)MAX_TILES * tile_of(s->dtype);
}

// The table entry nearest to a shape in (log2 B, log2(k + 1)) among those of
// its dtype and mode; nullptr when there is none.
inline const SvLayoutEntry *table_entry(const sv_shape_t *s) {
  const bool greedy = s->temperature == 0.f;
  double best = 1e30;
  const SvLayoutEntry *hit = nullptr;
  for (const SvLayoutEntry *e = kSvLayoutTable; e->dtype >= 0; ++e) {
    if (e->dtype != s->dtype || e->greedy != (greedy ? 1 : 0)) continue;
    const double db = log2((double)(s->B > 0 ? s->B : 1)) - log2((double)e->B);
    const double dk = log2((double)s->k + 1.0) - log2((double)e->k + 1.0);
    const double d = db * db + dk * dk;
    if (d < best) { best = d; hit = e; }
  }
  return hit;
}

// The item layout for a shape.  In launch order, tile c of every group goes
// to XCD (g * nT + c) mod 8, so with a tile count divisible by 4 the groups'
// last tiles, which run the merges, crowd onto 2 or 1 of the 8 XCDs (a 16-tile
// row measured 1.4x slower): XCD runs then.  Otherwise the measured table
// (taken at 19 bf16 and 38 fp32 tiles): the entry of the same dtype and mode
// nearest in (log2 B, log2(k + 1)); XCD runs where there is none.
inline int table_layout(const sv_shape_t *s) {
  const int nT = (s->V + tile_of(s->dtype) - 1) / tile_of(s->dtype);
  if (nT % 4 == 0) return SV_LAYOUT_XCD_RUNS;
  const SvLayoutEntry *e = table_entry(s);
  return e ? e->layout : SV_LAYOUT_XCD_RUNS;
}

// The kernel build for a shape: the nearest table entry's (bf16; fp32 has one).
inline int table_variant(const sv_shape_t *s) {
  if (s->dtype != SV_BF16) return SV_VARIANT_BASE;
  const SvLayoutEntry *e = table_entry(s);
  return e ? e->variant : SV_VARIANT_BASE;
}

// Every host-detectable argument check of spec_verify except the workspace,
// in the order the header lists them: SV_OK, or the code to return (SV_OK with
// *nothing = true when B == 0: nothing to enqueue).
inline int check_args(const sv_shape_t *shape, const void *target_logits, const void *draft_logits,
                      const int32_t *draft_tokens, const float *uniforms, const int32_t *accepted_len,
                      const int32_t *out_tokens, const float *topk_val, const int32_t *topk_idx, const sv_aux_t *aux,
                      bool *nothing) {
  *nothing = false;
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
  if (items + (int64_t)s.B * nT > 0x7fffffffLL || (int64_t)s.B * (s.k + 2) > 0x7fffffffLL) return SV_ERR_SHAPE;
  if (!(s.temperature >= 0.f) || s.temperature == INFINITY) return SV_ERR_TEMPERATURE;
  const bool greedy = s.temperature == 0.f;
  const int req_layout = aux ? aux->item_layout : SV_LAYOUT_AUTO;
  if (req_layout != SV_LAYOUT_AUTO && req_layout != SV_LAYOUT_LAUNCH && req_layout != SV_LAYOUT_XCD_RUNS)
    return SV_ERR_SHAPE;
  const int req_variant = aux ? aux->variant : SV_VARIANT_AUTO;
  if (req_variant != SV_VARIANT_AUTO && req_variant != SV_VARIANT_BASE && req_variant != SV_VARIANT_HIGH_OCC)
    return SV_ERR_SHAPE;
  if (s.B == 0) {
    *nothing = true;
    return SV_OK;
  }
  if (!target_logits || !accepted_len || !out_tokens || !topk_val || !topk_idx) return SV_ERR_NULL;
  if (s.k > 0 && !draft_tokens) return SV_ERR_NULL;
  if (!greedy && ((s.k > 0 && !draft_logits) || !uniforms)) return SV_ERR_NULL;
  return SV_OK;
}

// The workspace check: present, 256-byte aligned, large enough.
inline int check_workspace(const Layout &L, const void *workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;
  return SV_OK;
}

}  // namespace sv_host
