// moe_tuned.h -- the M-bucket tile table of the MoE-layer forward (included by moe_plan.h).
//
// One rule list per weight dtype (f32, bf16, fp8, and fp8 weights with fp8 activations): the
// first rule whose max_mean_rows is at least the problem's mean rows per routed expert (T*k/E)
// gives the m-tile size and the group size of the late phase's grouped item order.  Written by
// the tuner (python -m routed_grouped_gemm_amd.tune) from timings on the device:
//   bf16: d=2048 n=512 E=256 k=8, M in [16, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]
//   fp8: d=7168 n=2048 E=256 k=8, M in [1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096]
//   fp8a: d=7168 n=2048 E=256 k=8, M in [1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096]
#pragma once

namespace moe {
namespace {

struct TileRule {
  float max_mean_rows;  // upper bound (inclusive) of the bucket's mean rows per routed expert
  int m_tile_rows;      // 16, 32, 64, 128 or 160
  int group_m;          // late phase: m-tiles per group (m-tiles above 16 rows)
};

constexpr int kNumTileRules = 5;
constexpr TileRule kTileRules[4][kNumTileRules] = {
    // f32
    {{5.656854f, 16, 4}, {45.254834f, 64, 1}, {90.509668f, 128, 1}, {1e30f, 160, 4}, {1e30f, 160, 4}},
    // bf16
    {{5.656854f, 16, 4}, {45.254834f, 64, 1}, {90.509668f, 128, 1}, {1e30f, 160, 4}, {1e30f, 160, 4}},
    // fp8
    {{0.088388f, 16, 4}, {22.627417f, 32, 1}, {45.254834f, 64, 4}, {90.509668f, 128, 4}, {1e30f, 160, 1}},
    // fp8a
    {{0.088388f, 16, 4}, {45.254834f, 64, 1}, {90.509668f, 128, 4}, {1e30f, 160, 1}, {1e30f, 160, 1}},
};
constexpr const char *kTileTableSource = "tuned on the device";

}  // namespace
}  // namespace moe
