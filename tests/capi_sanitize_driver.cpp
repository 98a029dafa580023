// Host-side driver for the sanitizer build of the C ABI: every call below is
// one the library must answer without touching a GPU (size queries, argument
// and layer validation), run under AddressSanitizer and
// UndefinedBehaviorSanitizer with the library's own host code.  Sizes range
// from the ordinary to the extreme (negative, zero, INT_MAX) so that an
// overflowing size computation or an out-of-range read in the validation
// shows up as a sanitizer report.  Exit status 0 when every status matches.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <random>

#include "mxmoe.h"

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, long a, long b) {
  if (!ok) {
    std::printf("FAIL %s: got %ld expected %ld\n", what, a, b);
    ++g_fail;
  }
}
#define EXPECT_EQ(a, b) expect((long)(a) == (long)(b), #a, (long)(a), (long)(b))
#define EXPECT_TRUE(c) expect((c), #c, 0, 1)

// aligned non-null placeholders: validation never dereferences them
const void* P(uintptr_t v) { return reinterpret_cast<const void*>(v); }
template <class T>
T* Q(uintptr_t v) {
  return reinterpret_cast<T*>(v);
}

moe_layer_t layer(int H = 3072, int I = 1024, int E = 128, int k = 4, int Is = 1024) {
  moe_layer_t L{};
  L.hidden = H;
  L.inter = I;
  L.num_experts = E;
  L.top_k = k;
  L.shared_inter = Is;
  L.router_w = Q<const float>(0x10000);
  L.router_bias = nullptr;
  L.w13 = Q<const uint8_t>(0x10000);
  L.w13_scale = Q<const uint8_t>(0x10000);
  L.w2 = Q<const uint8_t>(0x10000);
  L.w2_scale = Q<const uint8_t>(0x10000);
  if (Is > 0) {
    L.ws13 = Q<const uint8_t>(0x10000);
    L.ws13_scale = Q<const uint8_t>(0x10000);
    L.ws2 = Q<const uint8_t>(0x10000);
    L.ws2_scale = Q<const uint8_t>(0x10000);
  }
  L.shared_folded = 0;
  L.norm_weight = nullptr;
  L.norm_eps = 0.f;
  return L;
}

void size_queries() {
  EXPECT_EQ(mx_codes_bytes(2048, 3072, MX_FMT_FP4, MX_LAYOUT_TILED), 2048 * 3072 / 2);
  EXPECT_EQ(mx_scales_bytes(2048, 3072, MX_LAYOUT_TILED), 128 * 6 * 256);
  EXPECT_EQ(mx_codes_bytes(4, 64, MX_FMT_FP4, MX_LAYOUT_TILED), 0);
  EXPECT_EQ(moe_align_sort_capacity(0, 4, 128, 64), 0);
  EXPECT_EQ(moe_align_sort_capacity(8192, 4, 128, 64), 32768 + 128 * 63);
  const int big = std::numeric_limits<int>::max();
  const int vals[] = {-big - 1, -1, 0, 1, 15, 16, 31, 32, 127, 128, 129, 4096, 65536, 1 << 20, big};
  for (int r : vals)
    for (int c : vals)
      for (int fmt = -1; fmt <= 2; ++fmt)
        for (int lay = -1; lay <= 2; ++lay) {
          (void)mx_codes_bytes(r, c, fmt, lay);
          (void)mx_scales_bytes(r, c, lay);
        }
  for (int T : vals)
    for (int k : {-1, 0, 1, 4, 8, 9, big})
      for (int E : {-1, 0, 1, 128, 256, 257, big})
        for (int bm : {-1, 0, 1, 64, 128, big}) {
          (void)moe_align_sort_capacity(T, k, E, bm);
          (void)moe_align_sort_workspace_bytes(T, k, E);
        }
}

void layer_validation() {
  const int big = std::numeric_limits<int>::max();
  moe_layer_t ok = layer();
  EXPECT_TRUE(moe_workspace_bytes(&ok, 16, 0) > 0);
  EXPECT_TRUE(moe_workspace_bytes(&ok, 64, 0) > moe_workspace_bytes(&ok, 16, 0));
  EXPECT_EQ(moe_workspace_bytes(&ok, 65, 0), 0);
  EXPECT_TRUE(moe_workspace_bytes(&ok, 8192, 1) > 0);
  EXPECT_EQ(moe_workspace_bytes(nullptr, 16, 0), 0);
  // one bad field at a time
  moe_layer_t bad[] = {layer(3000), layer(3072, 1000), layer(3072, 1024, 0), layer(3072, 1024, 300),
                       layer(3072, 1024, 128, 0), layer(3072, 1024, 128, 9), layer(3072, 1024, 2, 3),
                       layer(3072, 1024, 128, 4, 100), layer(-128), layer(big), layer(3072, big),
                       layer(3072, 1024, big), layer(3072, 1024, 128, big), layer(3072, 1024, 128, 4, big)};
  for (auto& L : bad) {
    EXPECT_EQ(moe_workspace_bytes(&L, 16, 0), 0);
    EXPECT_EQ(fused_moe_mxfp4_decode(&L, Q<const uint16_t>(0x20000), 1, nullptr, Q<uint16_t>(0x30000),
                                     Q<void>(0x20000), 1u << 30, nullptr, nullptr, nullptr),
              MOE_ERR_INVALID_ARGUMENT);
  }
  moe_layer_t nullw = layer();
  nullw.w13 = nullptr;
  EXPECT_EQ(moe_workspace_bytes(&nullw, 16, 0), 0);
  moe_layer_t misaligned = layer();
  misaligned.router_w = Q<const float>(0x10004);
  EXPECT_EQ(moe_workspace_bytes(&misaligned, 16, 0), 0);
  // folded shared expert
  moe_layer_t f = layer(3072, 1024, 128, 4, 0);
  f.shared_folded = 1;
  EXPECT_TRUE(moe_workspace_bytes(&f, 16, 0) > 0);
  f.top_k = 8;
  EXPECT_EQ(moe_workspace_bytes(&f, 16, 0), 0);
  f.top_k = 4;
  f.num_experts = 256;
  EXPECT_EQ(moe_workspace_bytes(&f, 16, 0), 0);
  moe_layer_t f2 = layer();
  f2.shared_folded = 1;  // with an MXFP8 shared expert as well
  EXPECT_EQ(moe_workspace_bytes(&f2, 16, 0), 0);
  // fused norm
  moe_layer_t n = layer();
  n.norm_weight = Q<const float>(0x50000);
  n.norm_eps = 1e-6f;
  EXPECT_TRUE(moe_workspace_bytes(&n, 16, 0) > 0);
  n.norm_eps = -1.f;
  EXPECT_EQ(moe_workspace_bytes(&n, 16, 0), 0);
  n.norm_eps = std::nanf("");
  EXPECT_EQ(moe_workspace_bytes(&n, 16, 0), 0);
  n.norm_eps = 1e-6f;
  n.norm_weight = Q<const float>(0x50004);
  EXPECT_EQ(moe_workspace_bytes(&n, 16, 0), 0);
  // random shapes: any combination must be answered without a sanitizer report
  std::mt19937 rng(1234);
  for (int it = 0; it < 20000; ++it) {
    auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
    moe_layer_t L = layer(pick({-128, 0, 128, 256, 1280, 3072, 8192, 1 << 20, big}),
                          pick({-128, 0, 128, 256, 384, 1024, 8192, 1 << 20, big}),
                          pick({-1, 0, 1, 2, 16, 128, 255, 256, 257, big}), pick({-1, 0, 1, 3, 4, 7, 8, 9, big}),
                          pick({-128, 0, 128, 256, 640, 1024, 8192, big}));
    L.shared_folded = pick({0, 0, 1, 2, -1});
    if (L.shared_folded == 1) {
      L.ws13 = L.ws13_scale = L.ws2 = L.ws2_scale = nullptr;
      L.shared_inter = 0;
    }
    for (int T : {-1, 0, 1, 4, 16, 17, 64, 65, 8192, 1 << 20, big})
      for (int path = -1; path <= 2; ++path) (void)moe_workspace_bytes(&L, T, path);
  }
}

void entry_point_errors() {
  moe_layer_t L = layer();
  const size_t n = moe_workspace_bytes(&L, 16, 0);
  const uint16_t* x = Q<const uint16_t>(0x20000);
  uint16_t* y = Q<uint16_t>(0x40000);
  void* ws = Q<void>(0x80000);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 65, nullptr, y, ws, n, nullptr, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 17, nullptr, y, ws, n, nullptr, nullptr, nullptr),
            MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 0, nullptr, y, ws, n, nullptr, nullptr, nullptr), MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, -5, nullptr, y, ws, n, nullptr, nullptr, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 4, nullptr, const_cast<uint16_t*>(x), ws, n, nullptr, nullptr, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, nullptr, 4, nullptr, y, ws, n, nullptr, nullptr, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 4, nullptr, y, Q<void>(0x80004), n, nullptr, nullptr, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_decode(&L, x, 4, nullptr, y, ws, n - 1, nullptr, nullptr, nullptr),
            MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(fused_moe_mxfp4_decode_noalloc(&L, x, 17, nullptr, y, nullptr, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT_EQ(fused_moe_mxfp4_decode_noalloc(&L, x, 0, nullptr, y, nullptr, nullptr, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_grouped(&L, x, 0, nullptr, y, ws, 1u << 30, nullptr), MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(fused_moe_mxfp4_grouped(&L, x, 8192, nullptr, y, ws, 16, nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(moe_router_topk(&L, x, 0, nullptr, Q<int32_t>(0x10000), Q<float>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(moe_router_topk(nullptr, x, 4, nullptr, Q<int32_t>(0x10000), Q<float>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(mx_quantize_weights(nullptr, 16, 128, 0, 1, Q<uint8_t>(0x10000), Q<uint8_t>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(mx_quantize_weights(Q<const float>(0x10000), 16, 100, 0, 1, Q<uint8_t>(0x10000), Q<uint8_t>(0x10000),
                                nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(mxfp4_quant_act(Q<const uint16_t>(0x10000), 4, 48, Q<uint8_t>(0x10000), Q<uint8_t>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(mx_requant_fp8_to_fp4(nullptr, Q<const uint8_t>(0x10000), 16, 128, 1, Q<uint8_t>(0x10000),
                                  Q<uint8_t>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(mx_requant_nvfp4_to_fp4(Q<const uint8_t>(0x10000), Q<const uint8_t>(0x10000), Q<const float>(0x10000),
                                    0, 16, 128, 1, Q<uint8_t>(0x10000), Q<uint8_t>(0x10000), nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(moe_align_sort(Q<const int32_t>(0x10000), 4, 2, 300, 1, Q<int32_t>(0x10000), Q<int32_t>(0x10000),
                           Q<int32_t>(0x10000), Q<int32_t>(0x10000), Q<void>(0x10000), 1u << 20, nullptr),
            MOE_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(moe_align_sort(Q<const int32_t>(0x10000), 4, 2, 8, 1, Q<int32_t>(0x10000), Q<int32_t>(0x10000),
                           Q<int32_t>(0x10000), Q<int32_t>(0x10000), Q<void>(0x10000), 4, nullptr),
            MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(moe_workspace_init(nullptr, 16, nullptr), MOE_ERR_INVALID_ARGUMENT);
  for (int code = -6; code <= 1; ++code) EXPECT_TRUE(moe_status_string((moe_status)code) != nullptr);
}

}  // namespace

int main() {
  size_queries();
  layer_validation();
  entry_point_errors();
  std::printf("%s: %d failures\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
