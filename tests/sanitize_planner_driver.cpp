// sanitize_planner_driver.cpp -- the host planner (fd_plan.cpp) over many
// shapes, extremes included, for a build with -fsanitize=address,undefined
// (tests/test_sanitizers.py).  Test infrastructure: undefined behaviour
// aborts the run; every accepted plan is checked for covering the whole
// sequence, a grid within the work list's bound, the merge rule and its
// workspace, and every rejection for being one of the defined codes.
#include <climits>
#include <cstdint>
#include <cstdio>

#include "fd_internal.h"

int main() {
  const int Bs[] = {1, 2, 7, 64, 130, 4096, 1 << 20};
  const int Hs[][2] = {{8, 8},  {64, 8}, {32, 32}, {16, 1},
                       {6, 2},  {256, 16}, {64, 2}, {128, 1}, {129, 1}};
  const int Ds[] = {64, 128, 96};
  const int Ls[] = {1, 31, 32, 33, 512, 513, 2048, 65536, 131072, 1 << 24,
                    (1 << 30) + 1, INT_MAX};
  const int Ss[] = {0, 1, 3, 7, 64, 4096, INT_MAX};
  const int cus[] = {1, 80, 256, 304};
  const int flag_sets[] = {0, FD_FLAG_FUSED_MERGE, FD_FLAG_PARTIALS,
                           FD_FLAG_UNIFIED_MAX,
                           FD_FLAG_FUSED_MERGE | FD_FLAG_PARTIALS};
  long plans = 0, rejected = 0, fails = 0, n = 0;
  for (int B : Bs)
    for (const auto &h : Hs)
      for (int D : Ds)
        for (int L : Ls)
          for (int S : Ss)
            for (int cu : cus) {
              ++n;
              const fd_dtype_t dt = (n % 3 == 0) ? FD_F32 : FD_BF16;
              const bool varlen = n % 2;
              const int flags = flag_sets[n % 5];
              const int variant = (int)(n % 7 % 3);
              fd::Extra ex;
              ex.Tq = (n % 11 == 0) ? 2 : 1;
              ex.paged = (n % 13 == 0);
              fd::Plan p{};
              const int rc = fd::make_plan(B, h[0], h[1], D, L, dt, varlen, S,
                                           variant, flags, cu, &p, ex);
              if (rc != FD_OK) {
                ++rejected;
                if (rc != FD_ERR_INVALID_ARG && rc != FD_ERR_UNSUPPORTED) {
                  std::printf("bad code %d\n", rc);
                  ++fails;
                }
                continue;
              }
              ++plans;
              const long long C = p.chunk, Sp = p.splits;
              const long long bound = (long long)B * h[1] * p.kv_rep * Sp;
              bool ok = C >= fd::kKeyTile && C % fd::kKeyTile == 0 && Sp >= 1 &&
                        Sp * C >= L && (Sp - 1) * C < L && p.grid >= 1 &&
                        p.grid <= bound && p.G * p.kv_rep == h[0] / h[1] && p.Hkv == h[1] * p.kv_rep &&
                        // virtual KV heads: vector-ALU half-groups, or
                        // matrix-core groups of more than 16 query rows
                        (p.kv_rep == 1 || p.variant == FD_VARIANT_VALU ||
                         (long)(h[0] / h[1]) * ex.Tq > fd::kMaxGroup) &&
                        (p.variant != FD_VARIANT_MFMA ||
                         (long)p.G * p.Tq <= fd::kMaxGroup) &&
                        // paged caches and several tokens: matrix cores only;
                        // the unified maximum: bf16 only
                        ((!ex.paged && ex.Tq == 1) ||
                         p.variant == FD_VARIANT_MFMA) &&
                        (!(flags & FD_FLAG_UNIFIED_MAX) || dt == FD_BF16) &&
                        p.combine == (Sp > 1 || (flags & FD_FLAG_PARTIALS)) &&
                        p.ws_bytes == fd::workspace_layout(p).total &&
                        (p.combine || p.ws_bytes == 0);
              if (S > 0 && !p.combine) ok = ok && Sp == 1;
              if (!ok) {
                ++fails;
                if (fails < 20)
                  std::printf("bad plan B=%d Hq=%d Hkv=%d D=%d L=%d S=%d cu=%d"
                              " -> chunk %d splits %d grid %d\n",
                              B, h[0], h[1], D, L, S, cu, p.chunk, p.splits,
                              p.grid);
              }
            }
  std::printf("plans %ld rejected %ld failures %ld\n", plans, rejected, fails);
  return fails ? 1 : 0;
}
