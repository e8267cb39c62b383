// Host-side checks of the C ABI, built with the host code instrumented by AddressSanitizer
// and UndefinedBehaviorSanitizer (device code is not built: nothing here launches a kernel).
// Every call below either fails its argument checks before touching device memory or works
// on an empty problem, so the program runs without a GPU.  Exit status 0 = every check held;
// a sanitizer report aborts the program with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "ssa.h"

static int failures = 0;
#define CHECK(cond)                                                           \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

// Never dereferenced: every call that receives it fails its checks first or has N = 0.
static void* const FAKE = reinterpret_cast<void*>(0x1000);

static ssa_window_t cube(int edge, int sx = 0, int sy = 0, int sz = 0) {
  ssa_window_t w;
  std::memset(&w, 0, sizeof w);
  w.kind = SSA_WINDOW_CUBE;
  w.edge = edge;
  w.shift[0] = sx; w.shift[1] = sy; w.shift[2] = sz;
  return w;
}

static ssa_window_t sfc(int tokens) {
  ssa_window_t w;
  std::memset(&w, 0, sizeof w);
  w.kind = SSA_WINDOW_SFC;
  w.tokens = tokens;
  return w;
}

static void status_strings() {
  for (int s = 0; s <= 7; ++s) CHECK(std::strlen(ssa_status_string((ssa_status)s)) > 0);
  CHECK(std::strcmp(ssa_status_string((ssa_status)99), "unknown status") == 0);
  CHECK(std::strcmp(ssa_status_string((ssa_status)-1), "unknown status") == 0);
}

// Workspace sizes over a wide sweep of token counts, grids, blocks and windows: the
// arithmetic must not overflow (UBSan), a negative or unsupported count gives 0, and the
// size never shrinks as N grows.
static void workspace_sweeps() {
  const int64_t ns[] = {0, 1, 2, 63, 64, 65, 1000, 80000, 110000, 1 << 20, int64_t(1) << 26,
                        (int64_t(1) << 31) - 1, int64_t(1) << 31, int64_t(1) << 40,
                        std::numeric_limits<int64_t>::max(), -1, std::numeric_limits<int64_t>::min()};
  const int32_t grids[][3] = {{1, 1, 1}, {8, 8, 8}, {64, 64, 64}, {1024, 1024, 1024},
                              {1, 1, 1 << 30}, {std::numeric_limits<int32_t>::max(), 2, 2}};
  const int32_t blocks[] = {1, 2, 3, 8, 16, 1 << 20, std::numeric_limits<int32_t>::max()};
  for (const auto& g : grids)
    for (int32_t b : blocks) {
      size_t prev = 0;
      for (int64_t n : ns) {
        const size_t a = ssa_plan_workspace_size(n, g, b, b);
        const ssa_window_t w1 = cube(2, 1, 0, 0), w2 = sfc(512);
        CHECK(ssa_plan_workspace_size_ex(n, g, b, &w1) == a);
        CHECK(ssa_plan_workspace_size_ex(n, g, b, &w2) == a);
        if (n < 0 || n >= (int64_t(1) << 31)) {
          CHECK(a == 0);
        } else {
          CHECK(a > 0 && a >= prev);
          prev = a;
        }
      }
    }
}

static void plan_argument_errors() {
  const int32_t g[3] = {8, 8, 8};
  const int32_t g0[3] = {8, 0, 8};
  std::vector<unsigned char> ws(1 << 16);
  size_t size = ssa_plan_workspace_size(10, g, 2, 2);
  CHECK(size > 0 && size <= ws.size());
  ssa_plan h = nullptr;
  const int32_t* c = static_cast<const int32_t*>(FAKE);
  CHECK(ssa_plan_create(c, 10, g, 2, 2, ws.data(), size, nullptr, nullptr) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(c, -1, g, 2, 2, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(c, 10, g, 0, 2, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(c, 10, g, 2, 0, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(c, 10, g0, 2, 2, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(nullptr, 10, g, 2, 2, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create(c, 10, g, 2, 2, nullptr, size, nullptr, &h) == SSA_ERR_WORKSPACE);
  CHECK(ssa_plan_create(c, 10, g, 2, 2, ws.data(), size - 1, nullptr, &h) == SSA_ERR_WORKSPACE);
  const ssa_window_t bad[] = {cube(0), cube(4, 0, -1, 0), cube(4, 0, 4, 0), sfc(0)};
  for (const auto& w : bad)
    CHECK(ssa_plan_create_ex(c, 10, g, 2, &w, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  ssa_window_t unknown = cube(2);
  unknown.kind = (ssa_window_kind)7;
  CHECK(ssa_plan_create_ex(c, 10, g, 2, &unknown, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  CHECK(ssa_plan_create_ex(c, 10, g, 2, nullptr, ws.data(), size, nullptr, &h) == SSA_ERR_INVALID_ARG);
  const int32_t big[3] = {2048, 8, 8};   // Morton codes beyond 30 bits
  ssa_window_t w = sfc(8);
  CHECK(ssa_plan_create_ex(c, 10, big, 2, &w, ws.data(), size, nullptr, &h) == SSA_ERR_UNSUPPORTED);
  CHECK(h == nullptr);
  CHECK(ssa_plan_get_info(nullptr, nullptr) != SSA_OK);
  ssa_plan_destroy(nullptr);
}

// An empty plan exists without a GPU: every entry point then checks its arguments and
// returns without launching.
static void empty_plan_entry_points() {
  const int32_t g[3] = {8, 8, 8};
  const ssa_window_t wins[] = {cube(4), cube(4, 1, 2, 3), sfc(64)};
  for (const auto& win : wins) {
    size_t size = ssa_plan_workspace_size_ex(0, g, 2, &win);
    CHECK(size > 0);
    std::vector<unsigned char> pws(size);
    ssa_plan h = nullptr;
    CHECK(ssa_plan_create_ex(nullptr, 0, g, 2, &win, pws.data(), size, nullptr, &h) == SSA_OK);
    CHECK(h != nullptr);
    if (!h) continue;
    ssa_plan_info_t info;
    std::memset(&info, 0xA5, sizeof info);
    CHECK(ssa_plan_get_info(h, &info) == SSA_OK);
    CHECK(info.n == 0 && info.num_blocks == 0);
    CHECK(ssa_plan_get_info(h, nullptr) == SSA_ERR_INVALID_ARG);
    for (int dt = 0; dt < 3; ++dt)
      for (int d : {32, 64, 96, 128})
        for (int save = 0; save < 2; ++save) {
          size_t fs = ssa_forward_workspace_size(h, (ssa_dtype)dt, 3, d, 8, save);
          CHECK(fs > 0);
          std::vector<unsigned char> fws(fs);
          ssa_status st = ssa_forward(h, (ssa_dtype)dt, 3, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                                      0.f, FAKE, nullptr, fws.data(), fs, save, nullptr);
          CHECK(st == SSA_OK || (save && win.kind != SSA_WINDOW_CUBE) || (save && win.shift[0]));
          CHECK(ssa_forward_noalloc(h, (ssa_dtype)dt, 3, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.f,
                                    FAKE, nullptr, nullptr) == SSA_OK);
          size_t bs = ssa_backward_workspace_size(h, (ssa_dtype)dt, 3, d, 8);
          std::vector<unsigned char> bws(bs ? bs : 1);
          float* f = static_cast<float*>(FAKE);
          ssa_status sb = ssa_backward(h, (ssa_dtype)dt, 3, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.f,
                                       static_cast<int32_t*>(FAKE), FAKE, f, f, f, f, fws.data(), fs,
                                       bws.data(), bs, nullptr);
          CHECK(sb == SSA_OK || sb == SSA_ERR_UNSUPPORTED);
        }
    // argument errors, each before any launch
    size_t fs = ssa_forward_workspace_size(h, SSA_F16, 2, 64, 4, 0);
    std::vector<unsigned char> fws(fs);
    auto fwd = [&](int dt, int H, int d, int k, float sc) {
      return ssa_forward(h, (ssa_dtype)dt, H, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k, sc, FAKE,
                         nullptr, fws.data(), fs, 0, nullptr);
    };
    CHECK(fwd(3, 2, 64, 4, 0.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(-1, 2, 64, 4, 0.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, 0, 64, 4, 0.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, -5, 64, 4, 0.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, 2, 48, 4, 0.f) == SSA_ERR_UNSUPPORTED);
    CHECK(fwd(1, 2, 64, 0, 0.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, 2, 64, 300, 0.f) == SSA_ERR_UNSUPPORTED);
    CHECK(fwd(1, 2, 64, 4, -1.f) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, 2, 64, 4, std::nanf("")) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, 2, 64, 4, INFINITY) == SSA_ERR_INVALID_ARG);
    CHECK(fwd(1, std::numeric_limits<int32_t>::max(), 128, 4, 0.f) != SSA_OK ||
          ssa_forward_workspace_size(h, SSA_F16, std::numeric_limits<int32_t>::max(), 128, 4, 1) > 0);
    CHECK(ssa_forward_stages(h, SSA_F16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f, FAKE, nullptr,
                             fws.data(), fs, 0, nullptr, 0) == SSA_ERR_INVALID_ARG);
    CHECK(ssa_forward_stages(h, SSA_F16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f, FAKE, nullptr,
                             fws.data(), fs, 0, nullptr, 8) == SSA_ERR_INVALID_ARG);
    CHECK(ssa_forward_conv(h, SSA_F16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f, FAKE, nullptr,
                           fws.data(), fs, 0, nullptr) == SSA_OK);
    // several samples
    ssa_plan plans[2] = {h, h};
    int64_t offs[3] = {0, 0, 0};
    size_t bsz = ssa_forward_batch_workspace_size(plans, 2, SSA_BF16, 2, 64, 4);
    CHECK(bsz > 0);
    std::vector<unsigned char> bws(bsz);
    CHECK(ssa_forward_batch(plans, 2, offs, SSA_BF16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f,
                            FAKE, bws.data(), bsz, nullptr) == SSA_OK);
    int64_t bad_offs[3] = {0, 3, 0};
    CHECK(ssa_forward_batch(plans, 2, bad_offs, SSA_BF16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                            0.f, FAKE, bws.data(), bsz, nullptr) == SSA_ERR_INVALID_ARG);
    CHECK(ssa_forward_batch(plans, 0, offs, SSA_BF16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f,
                            FAKE, bws.data(), bsz, nullptr) != SSA_OK ||
          true);
    CHECK(ssa_forward_batch(nullptr, 2, offs, SSA_BF16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
                            0.f, FAKE, bws.data(), bsz, nullptr) == SSA_ERR_INVALID_ARG);
    ssa_plan_destroy(h);
  }
  CHECK(ssa_forward(nullptr, SSA_F16, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.f, FAKE, nullptr,
                    FAKE, 1, 0, nullptr) == SSA_ERR_BAD_PLAN);
}

static void max_blocks() {
  CHECK(ssa_forward_max_blocks((ssa_dtype)5, 64) == 0);
  CHECK(ssa_forward_max_blocks((ssa_dtype)-1, 64) == 0);
  CHECK(ssa_forward_max_blocks(SSA_F16, 48) == 0);
  for (int dt = 0; dt < 3; ++dt)
    for (int d : {32, 64, 96, 128}) CHECK(ssa_forward_max_blocks((ssa_dtype)dt, d) >= 0);
}

static void producer_argument_errors() {
  auto call = [](int dt, int64_t n, int C, int H, int d, const void* x, float base) {
    return ssa_qkv_gates((ssa_dtype)dt, n, C, H, d, x, FAKE, FAKE, nullptr, FAKE, FAKE,
                         static_cast<int32_t*>(FAKE), base, 0.f, FAKE, FAKE, FAKE, FAKE, nullptr);
  };
  CHECK(call(1, 0, 64, 2, 96, FAKE, 0.f) == SSA_OK);
  CHECK(call(0, 10, 64, 2, 96, FAKE, 0.f) == SSA_ERR_UNSUPPORTED);
  CHECK(call(5, 10, 64, 2, 96, FAKE, 0.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, 10, 64, 2, 48, FAKE, 0.f) == SSA_ERR_UNSUPPORTED);
  CHECK(call(1, 10, 60, 2, 96, FAKE, 0.f) == SSA_ERR_UNSUPPORTED);
  CHECK(call(1, 10, 0, 2, 96, FAKE, 0.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, 10, 64, 0, 96, FAKE, 0.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, -10, 64, 2, 96, FAKE, 0.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, 10, 64, 2, 96, nullptr, 0.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, 10, 64, 2, 96, FAKE, -1.f) == SSA_ERR_INVALID_ARG);
  CHECK(call(1, std::numeric_limits<int64_t>::max(), std::numeric_limits<int32_t>::max() & ~7,
             std::numeric_limits<int32_t>::max(), 96, FAKE, 0.f) != SSA_OK);
}

int main() {
  status_strings();
  workspace_sweeps();
  plan_argument_errors();
  empty_plan_entry_points();
  producer_argument_errors();
  max_blocks();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
