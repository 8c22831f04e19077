// Fuzz driver for the host planner (ffa_plan.cpp), built by
// tests/test_plan_sanitizer_cpu.py with AddressSanitizer and
// UndefinedBehaviorSanitizer (g++, host code only; no HIP).
//
// The slice lists a caller passes to ffa_plan are untrusted input.  This
// driver feeds build_plan random problems -- all four mask types, invalid
// types, negative and reversed ranges, ranges past the axis, overlapping
// slices, empty slices, every head_dim, forced / automatic / no split, the
// backward worklists -- and checks that every call returns a documented
// status and that every accepted plan is internally consistent.  Any memory
// error, overflow or other undefined behaviour aborts the process under the
// sanitizers.
//
//   plan_fuzz <iterations> <seed>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../flexible_mask_flash_amd/csrc/ffa_internal.h"

namespace {

int fail(const char* what, int it) {
  std::fprintf(stderr, "plan_fuzz: %s (iteration %d)\n", what, it);
  return 1;
}

// Structural checks of an accepted plan: header, item and run records in range.
bool consistent(const ffa::Plan& p, int32_t total_q, int32_t total_k) {
  const int32_t* h = p.meta.data();
  if ((int64_t)p.meta.size() < ffa::kHdr) return false;
  if (h[ffa::kHdrMagic] != ffa::kMagic || h[ffa::kHdrItems] != p.num_items || h[ffa::kHdrRuns] != p.num_runs)
    return false;
  const int32_t* items = p.items();
  for (int32_t i = 0; i < p.num_items; ++i) {
    const int32_t* it = items + (size_t)i * ffa::kItemRec;
    const int32_t q0 = it[0], nrows = it[1], run_off = it[3], n_runs = it[4];
    if (q0 < 0 || nrows <= 0 || q0 + nrows > total_q) return false;
    if (n_runs < 0 || run_off < 0 || run_off + n_runs > p.num_runs) return false;
    int64_t tiles = 0;
    for (int32_t r = 0; r < n_runs; ++r) {
      const int32_t* rr = p.runs() + (size_t)(run_off + r) * ffa::kRec;
      const int32_t k0 = rr[0], nt = rr[1], nf = rr[2], nl = rr[5];
      if (nt <= 0 || nf < 0 || nl < 0 || nl + nf > nt || k0 < 0 || k0 >= total_k) return false;
      tiles += nt;
    }
    if (tiles != it[6]) return false;
  }
  return p.visible_pairs >= 0 && p.computed_pairs >= 0;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
  const unsigned seed = argc > 2 ? (unsigned)std::atoi(argv[2]) : 1u;
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int dims[] = {16, 32, 64, 128, 96, 0};
  int accepted = 0;
  for (int it = 0; it < iters; ++it) {
    const int32_t tq = uni(0, 1) ? uni(0, 700) : uni(-3, 40);
    const int32_t tk = uni(0, 1) ? uni(0, 900) : uni(-3, 40);
    const int32_t hkv = uni(0, 12) == 0 ? uni(-1, 0) : uni(1, 4);
    const int32_t hq = hkv > 0 ? hkv * uni(1, 8) + (uni(0, 15) == 0 ? 1 : 0) : uni(1, 4);
    const int32_t d = dims[uni(0, 5)];
    const int32_t ns = uni(0, 8);
    std::vector<int32_t> qr(2 * ns), kr(2 * ns), ty(ns);
    const bool disjoint = uni(0, 2) != 0;  // mostly valid problems, sometimes arbitrary ones
    int32_t qcur = 0;
    for (int s = 0; s < ns; ++s) {
      if (disjoint && tq > 0 && tk > 0) {
        // consecutive q bands, each with its own key range: never overlapping
        const int32_t a = std::min(qcur, tq), b = std::min(tq, a + uni(0, std::max(1, tq / 3)));
        qcur = b;
        const int32_t ka = uni(0, tk), kb = uni(ka, tk);
        qr[2 * s] = a; qr[2 * s + 1] = b; kr[2 * s] = ka; kr[2 * s + 1] = kb;
        ty[s] = uni(0, 3);
      } else {
        qr[2 * s] = uni(-5, tq + 5); qr[2 * s + 1] = uni(-5, tq + 5);
        kr[2 * s] = uni(-5, tk + 5); kr[2 * s + 1] = uni(-5, tk + 5);
        ty[s] = uni(-1, 5);
      }
    }
    const int32_t split = uni(0, 3) == 0 ? -1 : (uni(0, 1) ? 0 : uni(1, 20));
    const int32_t max_splits = uni(0, 4);
    const int32_t cus = uni(0, 20) == 0 ? uni(-1, 0) : uni(1, 256);
    const uint32_t flags = (uint32_t)uni(0, 3);
    ffa::Plan plan;
    const ffa_status st = ffa::build_plan(ns ? qr.data() : nullptr, ns ? kr.data() : nullptr,
                                          ns ? ty.data() : nullptr, ns, tq, tk, hq, hkv, d, split, max_splits, cus,
                                          flags, &plan);
    if (st < FFA_OK || st > FFA_ERR_ARG) return fail("status out of range", it);
    if (st == FFA_OK) {
      ++accepted;
      if (!consistent(plan, tq, tk)) return fail("inconsistent plan", it);
    }
  }
  // the long-context backward plan: one causal slice over 131072 tokens, Hq 64, Hkv 8
  {
    const int32_t T = 131072, qr[2] = {0, T}, kr[2] = {0, T}, ty[1] = {FFA_MASK_CAUSAL};
    ffa::Plan plan;
    if (ffa::build_plan(qr, kr, ty, 1, T, T, 64, 8, 128, 0, 0, 256, FFA_PLAN_BACKWARD, &plan) != FFA_OK)
      return fail("long-context backward plan rejected", -1);
    if (!consistent(plan, T, T)) return fail("long-context plan inconsistent", -1);
    if (plan.visible_pairs != (int64_t)T * (T + 1) / 2) return fail("long-context visible pairs", -1);
  }
  std::printf("plan_fuzz: %d iterations, %d plans accepted\n", iters, accepted);
  return accepted > 0 ? 0 : 1;
}
