// Calls every entry point of include/aware_tiling.h, with the launchers
// stubbed (api_stubs.cpp), over a grid of extreme arguments: negative, zero,
// boundary and INT64 extremes for the sizes, non-finite scales, null and
// misaligned pointers, short workspaces.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (any signed overflow or invalid access in the
// validation aborts the run).  Checks that a call launches only when it
// returns ATTN_OK (or ATTN_ERR_LAUNCH when the stub reports a HIP error),
// that null or misaligned pointers never launch, and that empty problems
// succeed without launching.  Prints "api validation: N calls" on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "aware_tiling.h"
#include <hip/hip_runtime.h>

extern int g_launches;
extern hipError_t g_launch_result;

static long g_calls = 0;

static void fail(const char* what, int line) {
  std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
  std::exit(1);
}
#define REQUIRE(c) \
  do {             \
    if (!(c)) fail(#c, __LINE__); \
  } while (0)

// Run one call; check the launch bookkeeping against the status.
template <class F>
static attn_status run(F f, bool pointers_ok) {
  const int before = g_launches;
  const attn_status s = f();
  ++g_calls;
  const bool launched = g_launches != before;
  REQUIRE(g_launches - before <= 1);
  if (launched) REQUIRE(pointers_ok);
  if (launched) REQUIRE(s == (g_launch_result == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH));
  if (s == ATTN_ERR_LAUNCH) REQUIRE(launched);
  REQUIRE(s >= ATTN_OK && s <= ATTN_ERR_LAUNCH);
  REQUIRE(attn_status_string(s) != nullptr);
  return s;
}

int main() {
  const int64_t BIG = std::numeric_limits<int64_t>::max(), SMALL = std::numeric_limits<int64_t>::min();
  const std::vector<int64_t> bhs = {-1, 0, 1, 3, (int64_t)1 << 20, ((int64_t)1 << 20) + 1, BIG, SMALL};
  const std::vector<int64_t> ns = {-1, 0, 1, 255, 4096, (int64_t)1 << 24, ((int64_t)1 << 24) + 1, BIG};
  const std::vector<int64_t> ds = {-1, 0, 64, 96, 128, 256, (int64_t)1 << 40, BIG, SMALL};
  const std::vector<float> scales = {0.125f, 0.0f, -1.0f, NAN, INFINITY};
  const std::vector<int64_t> extras = {-1, 0, 1, 2, 12288, 49152, 65536, 256, 257, BIG, SMALL};
  char* const base = reinterpret_cast<char*>(0x10000);
  const std::vector<void*> ptrs = {base, nullptr, base + 8};  // ok, null, misaligned
  const std::vector<size_t> wss = {0, 256, std::numeric_limits<size_t>::max()};

  for (hipError_t lr : {hipSuccess, hipErrorInvalidValue}) {
    g_launch_result = lr;
    for (int64_t bh : bhs)
      for (int64_t n : ns)
        for (int64_t d : ds)
          for (size_t pi = 0; pi < ptrs.size(); ++pi) {
            void* p = ptrs[pi];
            const bool pok = pi == 0;
            float* fp = static_cast<float*>(p);
            for (float sc : scales) {
              for (attn_dtype dt : {ATTN_BF16, ATTN_F32, (attn_dtype)7}) {
                run([&] { return attn_fwd(p, base, base, fp, nullptr, bh, n, d, sc, dt, nullptr); }, pok);
                run([&] { return attn_fwd_tile("default", p, base, base, fp, fp, bh, n, d, sc, dt, nullptr); }, pok);
              }
              run([&] { return attn_fwd_tile(nullptr, p, base, base, fp, fp, bh, n, d, sc, ATTN_BF16, nullptr); }, false);
              run([&] { return attn_fwd_tile("nope", p, base, base, fp, fp, bh, n, d, sc, ATTN_BF16, nullptr); }, false);
              for (int64_t x : extras) {
                run([&] { return attn_fwd_budget(p, base, base, fp, nullptr, bh, n, d, sc, ATTN_BF16, x, nullptr); }, pok);
                for (size_t w : wss) {
                  run([&] { return attn_fwd_splitk(p, base, base, fp, nullptr, bh, n, n < BIG - 7 ? n + 7 : n, d, sc, ATTN_BF16, x, base, w, nullptr); }, pok);
                  run([&] { return attn_fwd_splitk(p, base, base, fp, nullptr, bh, 1, n, d, sc, ATTN_BF16, x, base, w, nullptr); }, pok);
                  run([&] { return attn_fwd_smallcache(p, base, base, fp, nullptr, bh, n, d, sc, ATTN_BF16, x, base, w, nullptr); }, pok);
                  run([&] { return attn_bwd_smallcache(p, base, base, fp, base, fp, fp, fp, fp, bh, n, d, sc, ATTN_BF16, x, base, w, nullptr); }, pok);
                  run([&] { return attn_fwd_blocksparse(p, base, base, fp, nullptr, bh, n, d, sc, ATTN_BF16, reinterpret_cast<const uint8_t*>(base), x, base, w, nullptr); }, pok);
                }
                run([&] { return attn_fwd_splitk_noalloc(p, base, base, fp, nullptr, bh, n, n, d, sc, ATTN_BF16, x, nullptr); }, pok);
                (void)attn_fwd_splitk_splits(bh, n, x, d, x);
                (void)attn_fwd_splitk_workspace_size(bh, x, n, d, x);
                (void)attn_fwd_blocksparse_workspace_size(bh, n, x);
                (void)attn_fwd_smallcache_workspace_size(bh, n, d, x);
                (void)attn_bwd_smallcache_workspace_size(bh, n, d, x);
                (void)attn_smallcache_tile(d, x);
                (void)attn_bwd_smallcache_tile(d, x);
                (void)attn_bwd_smallcache_onchip_elems(d, x);
                (void)attn_smallcache_onchip_elems(x);
              }
              for (size_t w : wss) {
                run([&] { return attn_bwd(p, base, base, fp, base, fp, fp, fp, fp, bh, n, d, sc, ATTN_BF16, base, w, nullptr); }, pok);
                run([&] { return attn_bwd_tile("k256q256c64", p, base, base, fp, base, fp, fp, fp, fp, bh, n, d, sc, ATTN_BF16, base, w, nullptr); }, pok);
                run([&] { return attn_bwd_tile("nope", p, base, base, fp, base, fp, fp, fp, fp, bh, n, d, sc, ATTN_BF16, base, w, nullptr); }, false);
                run([&] { return attn_bwd_tile(nullptr, p, base, base, fp, base, fp, fp, fp, fp, bh, n, d, sc, ATTN_BF16, base, w, nullptr); }, false);
              }
            }
            (void)attn_bwd_workspace_size(bh, n, d);
            (void)attn_bwd_onchip_elems(d);
            (void)attn_fwd_onchip_elems(d, ATTN_BF16);
            (void)attn_fwd_query_block(d, ATTN_F32);
            (void)attn_fwd_budget_onchip_elems(d);
            int64_t a = 0, b = 0, c = 0;
            (void)attn_fwd_tile_info("default", d, &a, &b, &c);
            (void)attn_fwd_tile_info("nope", d, nullptr, nullptr, nullptr);
            (void)attn_fwd_tiles(d);
            (void)attn_bwd_tiles(d);
            (void)attn_bwd_tile_info("k256q256c64", d, &a, &b, &c, &a);
            (void)attn_bwd_tile_info("nope", d, nullptr, nullptr, nullptr, nullptr);
          }
    for (int64_t wg : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)INT32_MAX, (int64_t)INT32_MAX + 1, BIG})
      for (int32_t it : {-1, 0, 1, INT32_MAX})
        for (float amp : {1.0f, 0.0f, NAN, INFINITY})
          for (size_t pi = 0; pi < ptrs.size(); ++pi)
            run([&] { return attn_calib_mfma_loop(static_cast<float*>(ptrs[pi]), wg, it, amp, nullptr); }, pi == 0);
    for (int64_t wg : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)INT32_MAX / 256, (int64_t)INT32_MAX, BIG})
      for (int64_t nb : {(int64_t)-16, (int64_t)0, (int64_t)8, (int64_t)16, (int64_t)1 << 20, ((int64_t)1 << 20) + 4, BIG})
        for (size_t pi = 0; pi < ptrs.size(); ++pi)
          for (size_t po = 0; po < ptrs.size(); ++po)
            run([&] { return attn_calib_stream_read(ptrs[pi], nb, static_cast<uint32_t*>(ptrs[po]), wg, nullptr); },
                pi == 0 && po == 0);
  }
  // empty problems: success without a launch, even with null pointers
  g_launch_result = hipSuccess;
  const int before = g_launches;
  REQUIRE(attn_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 128, 64, 0.1f, ATTN_BF16, nullptr) == ATTN_OK);
  REQUIRE(attn_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 3, 0, 128, 0.1f, ATTN_BF16, nullptr) == ATTN_OK);
  REQUIRE(attn_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 64, 0.1f, ATTN_BF16, nullptr, 0, nullptr) == ATTN_OK);
  REQUIRE(g_launches == before);
  // one valid call of each kind does launch
  char* ws = base;
  REQUIRE(attn_fwd(base, base, base, reinterpret_cast<float*>(base), nullptr, 2, 300, 128, 0.1f, ATTN_BF16, nullptr) == ATTN_OK);
  REQUIRE(attn_bwd(base, base, base, reinterpret_cast<float*>(base), base, reinterpret_cast<float*>(base), reinterpret_cast<float*>(base), reinterpret_cast<float*>(base), reinterpret_cast<float*>(base), 2, 300, 128, 0.1f, ATTN_BF16, ws, 1 << 20, nullptr) == ATTN_OK);
  REQUIRE(g_launches == before + 2);
  std::printf("api validation: %ld calls\n", g_calls);
  return 0;
}
