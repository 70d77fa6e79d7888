// Host sanitizer driver for the planner (built with g++ -fsanitize=address,undefined
// by tests/test_host_sanitizers.py): random and edge-case descriptors through
// make_plan (weight gradient) and make_igemm_plan (forward, data gradient),
// checking the slice invariants of every accepted plan.  Any undefined
// behaviour (signed overflow, out-of-range shift, bad access) aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../implicit_gemm_amd/csrc/plan.h"

// The depthwise kernel's LDS size lives with the kernel (device code); a fixed
// plausible value is enough to drive the planner's arithmetic here.
int32_t cw::depthwise_lds_bytes(int32_t xl, int32_t R, int32_t S) {
  if (xl <= 0 || R <= 0 || S <= 0) return 0;
  return 48 * 1024;
}

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
int64_t pick(const int64_t* v, int n) { return v[next() % (uint64_t)n]; }

int check(const cw::Plan& p, const char* what) {
  const conv_wgrad_plan_t& q = p.pub;
  if (q.ks_count < 1 || q.units_per_slice < 1 || q.units < 1) return fprintf(stderr, "%s: empty plan\n", what), 1;
  if (p.dw_balanced) {
    // Depthwise slices balanced by staging steps: a boundary table from 0 to
    // the units, strictly increasing, whose longest slice is units_per_slice.
    if (q.ks_count > cw::Plan::kDwMaxSlices || p.dw_starts[0] != 0 || p.dw_starts[q.ks_count] != q.units)
      return fprintf(stderr, "%s: balanced slices do not cover the units\n", what), 1;
    int64_t longest = 0;
    for (int i = 0; i < q.ks_count; ++i) {
      const int64_t len = (int64_t)p.dw_starts[i + 1] - p.dw_starts[i];
      if (len < 1) return fprintf(stderr, "%s: empty balanced slice\n", what), 1;
      if (len > longest) longest = len;
    }
    if (longest != q.units_per_slice) return fprintf(stderr, "%s: balanced slice length\n", what), 1;
  } else if ((int64_t)(q.ks_count - 1) * q.units_per_slice >= q.units ||
             (int64_t)q.ks_count * q.units_per_slice < q.units) {
    return fprintf(stderr, "%s: slices do not cover the units exactly\n", what), 1;
  }
  if (q.grid != q.tiles * q.ks_count) return fprintf(stderr, "%s: grid\n", what), 1;
  if ((q.ks_count > 1) != (q.ws_bytes > 0)) return fprintf(stderr, "%s: workspace\n", what), 1;
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  const int64_t small[] = {1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 31, 32, 33, 64, 96, 127, 128, 255, 256, 384, 512};
  const int64_t big[] = {1, 3, 64, 1000, 65535, 65536, 1 << 20, (int64_t)1 << 30, (int64_t)1 << 31,
                         ((int64_t)1 << 31) - 1, (int64_t)1 << 40, INT64_MAX / 2, INT64_MAX, -1, 0};
  long accepted = 0, failures = 0;
  for (long it = 0; it < iters; ++it) {
    conv_wgrad_desc2_t d;
    memset(&d, 0, sizeof(d));
    const bool wild = next() % 8 == 0;
    const int64_t* pool = wild ? big : small;
    const int np = wild ? (int)(sizeof(big) / sizeof(big[0])) : (int)(sizeof(small) / sizeof(small[0]));
    d.N = pick(pool, np); d.C = pick(pool, np); d.H = pick(pool, np); d.W = pick(pool, np);
    d.K = pick(pool, np); d.R = 1 + (int64_t)(next() % 7); d.S = 1 + (int64_t)(next() % 7);
    if (wild && next() % 2) d.R = pick(pool, np);
    d.pad_h = (int64_t)(next() % 4); d.pad_w = (int64_t)(next() % 4);
    d.stride_h = 1 + (int64_t)(next() % 3); d.stride_w = 1 + (int64_t)(next() % 3);
    d.dil_h = 1 + (int64_t)(next() % 2); d.dil_w = 1 + (int64_t)(next() % 2);
    if (next() % 2) { d.pad_w = d.pad_h; d.stride_w = d.stride_h; d.dil_w = d.dil_h; }
    const int64_t gs[] = {1, 1, 1, 2, 4, 8, 16, 32, 64, 384};
    d.groups = gs[next() % 10];
    if (next() % 3 == 0) { d.C = d.groups * (1 + (int64_t)(next() % 8)); d.K = d.C; }
    d.dtype = (int32_t)(next() % 4) - (next() % 16 == 0 ? 1 : 0);
    const int32_t sks[] = {-1, -1, -1, 1, 2, 3, 7, 64, 1000, 65536, 0, -2};
    d.split_k = sks[next() % 12];
    d.math = (int32_t)(next() % 3);
    const int32_t fws[] = {-1, -1, 0, 1, 2, 4, 16};
    d.fold_width = fws[next() % 7];
    cw::Plan p;
    if (cw::make_plan(&d, &p) == CONV_WGRAD_OK) {
      ++accepted;
      failures += check(p, "wgrad");
    }
    for (int dir = CONV_DIRECTION_FWD; dir <= CONV_DIRECTION_DGRAD; ++dir)
      if (cw::make_igemm_plan(&d, dir, &p) == CONV_WGRAD_OK) failures += check(p, "igemm");
  }
  printf("plan_fuzz: %ld descriptors, %ld accepted, %ld failures\n", iters, accepted, failures);
  return failures ? 1 : 0;
}
