// Host planning code of the chunked forward (plan_host.h) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every sizing path over a grid of batch shapes,
// including empty, one-token, very long and packed batches, with invariants of
// the workspace layout checked on each. Exit status 0 when all hold.
#include <climits>
#include <cstdio>
#include <cstdlib>

#include "plan_host.h"

using namespace gla;

static int failures = 0;
#define CHECK(c)                                                                       \
  do {                                                                                 \
    if (!(c)) {                                                                        \
      std::fprintf(stderr, "plan_check: %s failed (B=%d T=%d H=%d dk=%d dv=%d N=%d C=%d cu=%d)\n", \
                   #c, B, T, H, dk, dv, N, C, (int)has_cu);                            \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

static void one(int B, int T, int H, int dk, int dv, int N, int C, bool has_cu, int n_cu,
                gla_dtype dt) {
  const int L = choose_seg_len(B, T, H, dk, dv, N, C, has_cu, n_cu, dt);
  CHECK(L >= C && L % C == 0 && L <= 65536);
  PlanLayout lay;
  const bool planned = make_plan(B, T, H, dk, dv, N, C, has_cu, n_cu, dt, lay);
  if (!planned) {
    CHECK(lay.total_bytes == 0);
    return;
  }
  CHECK(lay.seg_len == L);
  CHECK(lay.sub_len >= C && lay.sub_len % C == 0);
  CHECK(lay.n_sub >= 1 && (long)lay.n_sub * lay.sub_len >= lay.seg_len);
  CHECK(lay.max_items >= 0 && lay.max_state_items >= 0 && lay.max_multi >= 0 &&
        lay.max_slots >= 0);
  const size_t offs[] = {lay.off_header, lay.off_items, lay.off_state_items, lay.off_multi,
                         lay.off_slots, lay.off_slot_gamma, lay.total_bytes};
  for (int i = 0; i < 7; ++i) {
    CHECK(offs[i] % 256 == 0);
    if (i) CHECK(offs[i] >= offs[i - 1]);
  }
  CHECK(lay.off_slot_gamma - lay.off_slots >= sizeof(float) * (size_t)lay.max_slots * H * dk * dv);
}

int main() {
  const int shapes[][2] = {{64, 64}, {128, 128}, {64, 128}, {128, 64}, {96, 192}, {192, 96}};
  const int Ts[] = {0, 1, 63, 64, 65, 200, 2048, 4096, 65536, 1 << 20, INT_MAX / 64};
  const int Bs[] = {1, 2, 8, 64};
  const int Hs[] = {1, 2, 16, 32, 64};
  const int cus[] = {1, 80, 256, 304};
  for (const auto &sh : shapes)
    for (int T : Ts)
      for (int B : Bs)
        for (int H : Hs)
          for (int C : {64, 128})
            for (int n_cu : cus)
              for (gla_dtype dt : {GLA_BF16, GLA_F32})
                for (int cu = 0; cu < 2; ++cu) {
                  if ((long)B * T > INT_MAX) continue;
                  const bool has_cu = cu == 1;
                  const int Bx = has_cu ? 1 : B, N = has_cu ? B : B;
                  one(Bx, T, H, sh[0], sh[1], N, C, has_cu, n_cu, dt);
                }
  // overlap test: adjacent, nested, disjoint, empty
  char buf[64];
  const int B = 0, T = 0, H = 0, dk = 0, dv = 0, N = 0, C = 0;
  const bool has_cu = false;
  CHECK(!overlaps(buf, 16, buf + 16, 16));
  CHECK(overlaps(buf, 17, buf + 16, 16));
  CHECK(overlaps(buf, 64, buf + 8, 8));
  CHECK(!overlaps(buf, 0, buf, 8));
  CHECK(!overlaps(nullptr, 8, buf, 8));
  std::printf("plan_check: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
