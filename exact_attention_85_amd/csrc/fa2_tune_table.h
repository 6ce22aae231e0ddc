// Forward configuration per shape class: the rows fa2_fwd and fa2_fwd_window
// look up (the synthesis page, section 3 item 3 and section 5 item 1: block
// sizes, warp counts and similar launch choices searched per shape instead of
// a few hand-picked ones).  Written by exact_attention_85_amd/tune.py from its
// measurements; tune.py --write replaces this file.
//
// Each row: head dim, banded (causal or windowed), the smallest N_q the row
// applies to, and the configuration (index into kFwdConfigs).  For a shape the
// row with matching d and banded and the largest nq_min <= N_q applies.
#pragma once

namespace fa2 {

struct TuneRow {
  int d;
  int banded;
  int nq_min;
  int config;
};

// source: tune.py on AMD Radeon Graphics (256 CUs), 2026-12-03 07:33 UTC, 15 reps
constexpr TuneRow kTuneTable[] = {
    {64, 0, 1, 8},  // tile256_remap_headmajor
    {64, 1, 1, 9},  // tile256_noremap_qbmajor
    {128, 0, 1, 0},  // tile128_remap_headmajor
    {128, 0, 1448, 4},  // pingpong256_remap_headmajor
    {128, 1, 1, 9},  // tile256_noremap_qbmajor
    {128, 1, 2896, 7},  // pingpong256_noremap_qbmajor
};

}  // namespace fa2
