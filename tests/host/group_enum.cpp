// Host-only driver for the library's argument checks and group addressing.
// Built with g++ by the CPU tests; prints every token group a launch would use
// so that the test can compare them with the oracle's token sets.
//
//   group_enum groups T H W r_axes tile_t tile_h   -> "R g: tokens" / "L g: tokens" lines
//   group_enum remap n_max                          -> "ok" if xcd_remap is a bijection for all n
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../structured_attention_video_attn_amd/csrc/validate.h"

static void dump(const char *tag, const GroupAddr &a) {
  for (int32_t g = 0; g < a.n_groups; ++g) {
    GroupGeom gg = group_geom(a, g);
    std::printf("%s %d:", tag, g);
    for (int32_t m = 0; m < gg.len; ++m) std::printf(" %d", member_token(gg, m));
    std::printf("\n");
  }
}

int main(int argc, char **argv) {
  if (argc >= 2 && std::strcmp(argv[1], "remap") == 0) {
    const uint32_t n_max = (uint32_t)std::atoi(argv[2]);
    for (uint32_t n = 1; n <= n_max; ++n) {
      std::vector<char> seen(n, 0);
      for (uint32_t b = 0; b < n; ++b) {
        uint32_t l = xcd_remap(b, n);
        if (l >= n || seen[l]) { std::printf("bad n=%u b=%u\n", n, b); return 1; }
        seen[l] = 1;
      }
    }
    std::printf("ok\n");
    return 0;
  }
  if (argc != 8 || std::strcmp(argv[1], "groups") != 0) return 2;
  int T = std::atoi(argv[2]), H = std::atoi(argv[3]), W = std::atoi(argv[4]);
  int r_axes = std::atoi(argv[5]), tt = std::atoi(argv[6]), th = std::atoi(argv[7]);
  ma::Problem p;
  const bool tiled = tt != 0 || th != 0;
  int st = ma::resolve_grid(1, 1, T, H, W, r_axes, tt, th, tiled, 16, MA_F32, &p);
  if (st != MA_OK) { std::printf("status %d\n", st); return 0; }
  std::printf("trivial %d %d\n", (int)p.r_trivial, (int)p.l_trivial);
  dump("R", ma::stage_r_groups(p));
  dump("L", ma::stage_l_groups(p));
  return 0;
}
