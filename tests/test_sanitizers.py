"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (every
finding aborts: -fno-sanitize-recover=all).

  * The library's host-side argument checks, workspace layout and item-layout
    lookup (draft_verification_spec_amd/csrc/sv_host.h, the code spec_verify
    runs before it enqueues anything), built with g++ and driven over valid and
    invalid shapes, strides, temperatures, layouts and null pointers.
  * The C oracles (oracle/sv_oracle.c, oracle/kd_oracle.c), built with gcc and
    driven over small random batches and the data-error cases: NaN, +inf and
    all -inf rows, tokens and uniforms out of range, V = 1, k = 0, greedy,
    padding, repeated and out-of-range stored ids.
No GPU is involved; nothing here is loaded by the product path.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")

HOST_DRIVER = r"""
#include <stdio.h>
#include "sv_host.h"
using namespace sv_host;

static char mem[4096];                     // pointers handed to the checks, never dereferenced

int main() {
  const int Bs[] = {-1, 0, 1, 2, 7, 32, 256, 4096, 2000000000};
  const int ks[] = {-1, 0, 1, 3, 8, 15, 63, 64, 70, 260};
  const int Vs[] = {0, 1, 7, 31, 32, 1000, 4097, 128256, 151936, 262144, 262145, 524288, 524289};
  const int dts[] = {0, 1, 7};
  const float Ts[] = {__builtin_nanf(""), -1.f, 0.f, 0.7f, 1.f, __builtin_inff()};
  const long long strides[] = {0, -5, 1, 200000};
  const int lays[] = {0, 1, 2, 3, -1};
  long long valid = 0, rejected = 0;
  for (int B : Bs) for (int k : ks) for (int V : Vs) for (int dt : dts) for (float T : Ts)
    for (long long st : strides) for (int lay : lays) for (int nulls = 0; nulls < 3; ++nulls) {
      sv_shape_t s = {B, k, V, dt, st, st, T};
      sv_aux_t aux = {};
      aux.item_layout = lay;
      void *p = mem;
      const void *d = nulls == 1 ? nullptr : p;        // draft logits missing
      const float *u = nulls == 2 ? nullptr : (const float *)p;
      bool nothing = false;
      const int rc = check_args(&s, p, d, (const int32_t *)p, u, (const int32_t *)p, (const int32_t *)p,
                                (const float *)p, (const int32_t *)p, &aux, &nothing);
      if (rc != SV_OK || nothing) { ++rejected; continue; }
      ++valid;
      const Layout L = layout_for(B, k, V, dt);
      const size_t offs[] = {L.fault, L.garrive, L.sarrive, L.ddone, L.recs, L.grec, L.srec, L.cand,
                             L.dtot, L.total};
      for (int i = 0; i < 10; ++i) {
        if (offs[i] % 256) { printf("unaligned section %d\n", i); return 1; }
        if (i && offs[i] < offs[i - 1]) { printf("sections out of order\n"); return 1; }
      }
      if (check_workspace(L, mem + 256 - ((unsigned long)mem & 255), L.total) != SV_OK &&
          ((unsigned long)mem & 255) == 0) { printf("workspace rejected\n"); return 1; }
      if (check_workspace(L, nullptr, L.total) != SV_ERR_WORKSPACE) { printf("null workspace\n"); return 1; }
      if (L.total && check_workspace(L, (void *)256, L.total - 1) != SV_ERR_WORKSPACE) { printf("short\n"); return 1; }
      if (check_workspace(L, (void *)1, L.total) != SV_ERR_WORKSPACE) { printf("misaligned\n"); return 1; }
      const int tl = table_layout(&s);
      if (tl != SV_LAYOUT_LAUNCH && tl != SV_LAYOUT_XCD_RUNS) { printf("layout %d\n", tl); return 1; }
    }
  bool nothing = false;
  if (check_args(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, &nothing) != SV_ERR_NULL) return 1;
  printf("valid %lld rejected %lld\n", valid, rejected);
  return valid > 0 && rejected > 0 ? 0 : 1;
}
"""

ORACLE_DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_verify(int B, int k, int V, int dtype, float temperature, const void *target, const void *draft,
               const int32_t *tokens, const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
               float *topk_val, int32_t *topk_idx, int32_t *status, double *lse_target, double *lse_draft,
               double *p_tok, double *q_tok, double *margin_accept, double *margin_cdf);
int kd_oracle(int N, int V, int dtype, int64_t stride, int S, int group, double w_max, const void *logits,
              const float *tval, const int32_t *tidx, const int32_t *row_sample, const float *rewards, double *kl,
              double *weight, int32_t *status, double *loss, double *grad);

static uint32_t rng = 12345u;
static float unif(void) { rng = rng * 1664525u + 1013904223u; return (float)(rng >> 8) / 16777216.0f; }

static int run_verify(int B, int k, int V, int dtype, float T, int plant) {
  const size_t e = dtype ? 2 : 4;
  const int K1 = k + 1;
  char *t = malloc((size_t)B * K1 * V * e + 1), *d = malloc((size_t)B * (k ? k : 1) * V * e + 1);
  int32_t *tok = malloc(sizeof(int32_t) * (size_t)B * (k ? k : 1));
  float *u = malloc(sizeof(float) * (size_t)B * (k + 2));
  for (size_t i = 0; i < (size_t)B * K1 * V; ++i) {
    const float x = 4.f * (unif() - 0.5f);
    if (dtype) { uint32_t b; memcpy(&b, &x, 4); ((uint16_t *)t)[i] = (uint16_t)(b >> 16); }
    else ((float *)t)[i] = x;
  }
  for (size_t i = 0; i < (size_t)B * k * V; ++i) {
    const float x = 4.f * (unif() - 0.5f);
    if (dtype) { uint32_t b; memcpy(&b, &x, 4); ((uint16_t *)d)[i] = (uint16_t)(b >> 16); }
    else ((float *)d)[i] = x;
  }
  for (int i = 0; i < B * k; ++i) tok[i] = (int32_t)(unif() * V);
  for (int i = 0; i < B * (k + 2); ++i) u[i] = unif();
  if (plant && B > 0) {                                /* the data errors, one per sequence */
    const float nan = NAN, pinf = INFINITY, ninf = -INFINITY;
    for (int x = 0; x < V && dtype == 0; ++x) {
      if (B > 1) ((float *)t)[(size_t)1 * K1 * V + x] = ninf;          /* an all -inf target row */
    }
    if (dtype == 0) ((float *)t)[0] = nan;
    if (dtype == 0 && B > 2) ((float *)t)[(size_t)2 * K1 * V + 1] = pinf;
    if (k > 0 && B > 3) tok[3 * k] = V;                /* a token out of range */
    if (B > 4) u[4 * (k + 2)] = 1.0f;                  /* a uniform out of range */
  }
  int32_t *acc = malloc(sizeof(int32_t) * (size_t)B + 4), *out = malloc(sizeof(int32_t) * (size_t)B * K1 + 4);
  float *tv = malloc(sizeof(float) * (size_t)B * K1 * 32 + 4);
  int32_t *ti = malloc(sizeof(int32_t) * (size_t)B * K1 * 32 + 4), *st = malloc(sizeof(int32_t) * (size_t)B + 4);
  double *lt = malloc(sizeof(double) * (size_t)B * K1 + 8), *ld = malloc(sizeof(double) * (size_t)B * (k ? k : 1));
  double *pt = malloc(sizeof(double) * (size_t)B * (k ? k : 1)), *qt = malloc(sizeof(double) * (size_t)B * (k ? k : 1));
  double *ma = malloc(sizeof(double) * (size_t)B * (k ? k : 1)), *mc = malloc(sizeof(double) * (size_t)B + 8);
  const int rc = orc_verify(B, k, V, dtype, T, t, T == 0.f ? NULL : d, tok, T == 0.f ? NULL : u, acc, out, tv, ti,
                            st, lt, ld, pt, qt, ma, mc);
  free(t); free(d); free(tok); free(u); free(acc); free(out); free(tv); free(ti); free(st);
  free(lt); free(ld); free(pt); free(qt); free(ma); free(mc);
  return rc;
}

static int run_kd(int N, int V, int dtype) {
  const size_t e = dtype ? 2 : 4;
  char *z = malloc((size_t)N * V * e);
  for (size_t i = 0; i < (size_t)N * V; ++i) {
    const float x = 3.f * (unif() - 0.5f);
    if (dtype) { uint32_t b; memcpy(&b, &x, 4); ((uint16_t *)z)[i] = (uint16_t)(b >> 16); }
    else ((float *)z)[i] = x;
  }
  float *tv = malloc(sizeof(float) * (size_t)N * 32), rw[4] = {1.0f, 0.5f, 0.0f, 0.0f};
  int32_t *ti = malloc(sizeof(int32_t) * (size_t)N * 32), *rs = malloc(sizeof(int32_t) * (size_t)N);
  for (int n = 0; n < N; ++n) {
    rs[n] = n % 4;
    for (int j = 0; j < 32; ++j) { tv[n * 32 + j] = 5.f * unif(); ti[n * 32 + j] = j % V; }
  }
  if (N > 1) ti[1 * 32 + 5] = ti[1 * 32 + 6];          /* a repeated id */
  if (N > 2) { tv[2 * 32 + 3] = -INFINITY; ti[2 * 32 + 4] = -1; }   /* padding */
  if (N > 3) ti[3 * 32 + 7] = V + 3;                   /* an id out of range */
  if (N > 4) rs[4] = 9;                                /* a sample out of range */
  if (N > 5) tv[5 * 32] = NAN;
  double *kl = malloc(sizeof(double) * N), *w = malloc(sizeof(double) * N), loss = 0;
  int32_t *st = malloc(sizeof(int32_t) * N);
  double *g = malloc(sizeof(double) * (size_t)N * V);
  const int rc = kd_oracle(N, V, dtype, V, 4, 2, 0.75, z, tv, ti, rs, rw, kl, w, st, &loss, g);
  free(z); free(tv); free(ti); free(rs); free(kl); free(w); free(st); free(g);
  return rc;
}

int main(void) {
  int bad = 0;
  const int Vs[] = {1, 2, 7, 33, 300};
  for (int vi = 0; vi < 5; ++vi)
    for (int k = 0; k <= 3; ++k)
      for (int dt = 0; dt < 2; ++dt)
        for (int plant = 0; plant < 2; ++plant) {
          bad |= run_verify(6, k, Vs[vi], dt, 1.0f, plant);
          bad |= run_verify(6, k, Vs[vi], dt, 0.0f, plant);
          bad |= run_verify(6, k, Vs[vi], dt, 0.7f, plant);
        }
  bad |= run_verify(0, 3, 10, 0, 1.0f, 0);
  bad |= run_verify(2, 70, 20, 1, 1.0f, 0) != 0;
  for (int dt = 0; dt < 2; ++dt) bad |= run_kd(8, 40, dt) | run_kd(3, 20, dt) | run_kd(6, 1, dt);
  printf("oracle runs done, bad=%d\n", bad);
  return bad;
}
"""


def _build_and_run(tmp_path, name, compiler, src_text, ext, extra_srcs, includes=()):
    src = tmp_path / f"{name}.{ext}"
    src.write_text(src_text)
    exe = tmp_path / name
    cmd = [compiler, *SAN, *[f"-I{i}" for i in includes], "-o", str(exe), str(src), *extra_srcs, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_host_checks_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "host_checks", "g++", HOST_DRIVER, "cpp", [],
                         includes=[os.path.join(ROOT, "draft_verification_spec_amd", "csrc"),
                                   os.path.join(ROOT, "include")])
    assert "valid" in out


def test_oracles_under_sanitizers(tmp_path):
    srcs = [os.path.join(ROOT, "oracle", "sv_oracle.c"), os.path.join(ROOT, "oracle", "kd_oracle.c")]
    out = _build_and_run(tmp_path, "oracle_runs", "gcc", ORACLE_DRIVER, "c", srcs)
    assert "bad=0" in out
