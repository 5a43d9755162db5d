// fr_plan.hip -- the launch planner (host code): which variant, how many
// waves per workgroup, row blocks and key splits a call runs with, and the
// device workspace it needs.  Kept apart from the C-ABI glue so that the
// kernels and their plan can be tracked together.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "fr_decode_attn.h"
#include "fr_internal.h"

namespace fr {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups the split kernel should launch to cover the machine: 256 compute
// units on MI355X, one resident workgroup per unit at these LDS sizes.
constexpr int kTargetWorkgroups = 256;

int make_plan(int n_inst, int n_head, int n_tok, int n_kv, int hd, unsigned flags,
              Plan *plan) {
  Plan p;
  const int M = n_head * n_tok;
  const bool unmasked = (flags & FR_PLAN_UNMASKED) != 0;
  p.variant = (flags & FR_VARIANT_DECOMPOSED) ? kDecomposed : kFused;
  const int tiles_total = (int)cdiv(M, 16);
  if (p.variant == kDecomposed) {
    // QK^T and PV kernels: 4 waves, a fixed number of 16-row tiles per wave
    p.waves = 4;
    p.tiles = hd == 256 ? 1 : (hd == 128 ? 2 : 4);   // hd 64 and 80: 4
  } else {
    // split kernel: one 16-row tile per wave.  Up to 16 tiles run as row
    // blocks of 4 waves (one per SIMD, 64 rows per workgroup): small row
    // blocks keep each workgroup's query loads and partial stores short and
    // spread the call over more compute units.  More rows use 8 waves (two per
    // SIMD, hiding each other's latency), which halves how often the K/V
    // blocks are staged per row.
    p.waves = tiles_total <= 16 ? 4 : 8;
    p.tiles = 1;
    // An unmasked call with many rows (a prefill): its 4-wave row blocks alone
    // nearly fill the machine, so few key splits are needed and the partials
    // (and their combine) shrink (968-token prefill: 38 -> 33 us per call).
    if (unmasked && (int64_t)n_inst * cdiv(tiles_total, 4) >= 64) p.waves = 4;
    const int fw = env_int("FR_FORCE_WAVES", 0);   // developer knob (tests, A/B timing)
    if (fw == 4 || fw == 8) p.waves = fw;
    // more query tokens than a 4-wave workgroup stages mask rows for
    if (!unmasked && n_tok > max_tokens(4)) p.waves = 8;
  }
  const int key_blocks = (int)cdiv(n_kv, kKeyBlock);
  const int forced = env_int("FR_FORCE_SPLITS", 0);
  // Row blocks of at most tiles_cap tiles, balanced: with 5 tiles and room
  // for 4, blocks of 3 and 2 rather than 4 and 1 (the largest block sets the
  // per-workgroup query loads and partial stores).  Key splits: as many as
  // keep the grid within one workgroup per compute unit.  Where that leaves a
  // single key block per split, two blocks per split are taken instead if the
  // grid still covers half the machine: the partials (and their combine) then
  // halve, and block 1 loads while block 0 is computed.
  auto decompose = [&](int tiles_cap) {
    p.n_rowblk = (int)cdiv(tiles_total, tiles_cap);
    p.tpr = p.variant == kFused ? (int)cdiv(tiles_total, p.n_rowblk) : tiles_cap;
    const int64_t wg_per_split = (int64_t)n_inst * p.n_rowblk;
    int want = (int)std::max<int64_t>(1, kTargetWorkgroups / wg_per_split);
    if (cdiv(key_blocks, want) < 2 && wg_per_split * cdiv(key_blocks, 2) >= kTargetWorkgroups / 2)
      want = (int)cdiv(key_blocks, 2);
    if (forced > 0) want = forced;
    want = std::min(std::max(want, 1), key_blocks);
    const int blocks_per_split = (int)cdiv(key_blocks, want);
    p.chunk = blocks_per_split * kKeyBlock;
    p.n_split = (int)cdiv(key_blocks, blocks_per_split);
    p.grid = n_inst * p.n_rowblk * p.n_split;
  };
  decompose(p.waves * p.tiles);
  // Where the key blocks cap the splits and row blocks of four tiles leave the
  // grid below three quarters of the machine (the f16-Q workload: 128
  // workgroups; the causal tail: 64), row blocks of at most two tiles double
  // the grid and halve each workgroup's query loads and partial stores (its
  // other waves only stage K/V): f16-Q 11.0 -> 10.4 us per call, causal tail
  // 12.4 -> 11.5.  Row blocks of one tile, or this rule on the pi0.5 step's
  // 216 workgroups, were slower.
  if (p.variant == kFused && p.waves == 4 && p.tiles == 1 && p.grid < 3 * kTargetWorkgroups / 4 &&
      env_int("FR_FORCE_WAVES", 0) == 0) {
    const Plan four = p;
    decompose(2);
    if (p.grid > kTargetWorkgroups) p = four;   // only while the grid still fits the machine
  }
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t rows = (size_t)n_inst * p.n_split * M;
  if (p.variant == kFused) {
    p.launches = p.n_split > 1 ? 2 : 1;
    p.ws_bytes = p.n_split > 1 ? al(rows * hd * sizeof(float) + rows * 2 * sizeof(float)) : 0;
  } else {
    // [PV partials when split] [scores fp32 M x kv_pad] [probabilities f16 M x kv_pad]
    // [probability sums fp32 M]
    const size_t kv_pad = (size_t)key_blocks * kKeyBlock;
    p.launches = 3 + (p.n_split > 1 ? 1 : 0);
    p.ws_bytes = (p.n_split > 1 ? al(rows * hd * sizeof(float)) : 0) +
                 al((size_t)n_inst * M * kv_pad * sizeof(float)) +
                 al((size_t)n_inst * M * kv_pad * sizeof(uint16_t)) +
                 al((size_t)n_inst * M * sizeof(float));
  }
  *plan = p;
  return FR_OK;
}

}  // namespace fr
