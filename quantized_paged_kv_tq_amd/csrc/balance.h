// Balanced work partition of the INT4 decode, shared by stage 1 (which
// produces the partials) and stage 2 (which finds them).
//
// The split ranges are those of the TurboQuant stage 1
// (triton_turboquant_decode.py, _tq_decode_stage1): split_len = ceil(seq/S),
// split s covers [s*split_len, min((s+1)*split_len, seq)), empty splits are
// skipped. Each split is cut into tiles of 64 tokens (the last tile of a
// split may be shorter). The tiles of all sequences, in (sequence, split,
// tile) order, form one list of N tiles per kv-head group; workgroup w of
// nw takes the contiguous range [w*N/nw, (w+1)*N/nw), so every workgroup
// streams the same number of tiles whatever the mix of sequence lengths.
//
// A split that lies inside one range is written to its own partial slot
// ws[b, h, s]. A split cut by range boundaries leaves one piece per range it
// touches, each in a piece slot of that workgroup: slot 0 for the range's
// first split, slot 1 for its last split (a range cuts at most these two).
// Stage 2 merges whole splits and pieces alike by log-sum-exp.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tqk {

constexpr int kTileTokens = 64;
// Waves the balanced INT4 decode keeps in flight: 8 per CU on 256 CUs.
constexpr int kWaveBudget = 2048;

struct SeqSplits {
  int seq;    // sequence length, clamped to the block-table capacity
  int L;      // split length ceil(seq / S)
  int n;      // non-empty splits ceil(seq / L)
  int TL;     // tiles of a full split
  int TLast;  // tiles of the last split
};

__device__ __forceinline__ SeqSplits seq_splits(const DecodeParams& p, int b) {
  int64_t s64 = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  s64 = s64 < 0 ? 0 : (s64 > cap ? cap : s64);
  SeqSplits r;
  r.seq = (int)s64;
  if (r.seq == 0) {
    r.L = r.n = r.TL = r.TLast = 0;
    return r;
  }
  r.L = (r.seq + p.splits - 1) / p.splits;
  r.n = (r.seq + r.L - 1) / r.L;
  r.TL = (r.L + kTileTokens - 1) / kTileTokens;
  r.TLast = (r.seq - (r.n - 1) * r.L + kTileTokens - 1) / kTileTokens;
  return r;
}

__device__ __forceinline__ int seq_tiles(const SeqSplits& q) {
  return q.n ? (q.n - 1) * q.TL + q.TLast : 0;
}

// First tile of workgroup w's range (N tiles over nw workgroups).
__device__ __forceinline__ int range_lo(int w, int N, int nw) {
  return (int)((int64_t)w * N / nw);
}
// The workgroup whose range holds tile x (0 <= x < N): the largest w with
// range_lo(w) <= x.
__device__ __forceinline__ int range_owner(int x, int N, int nw) {
  return (int)(((int64_t)(x + 1) * nw - 1) / N);
}

// Kv heads per workgroup and workgroups per kv-head group of the balanced
// layout (host side; the piece region is sized by the default rule). A wave
// serves four query heads of one kv head, so a kv head with g query heads
// takes ceil(g / 4) waves (a layout whose waves serve all of a kv head's
// query heads passes g = 4); a workgroup has at most max_waves waves and
// the grid at most `budget`.
inline int balance_heads_per_wg(int hk, int g, int max_waves = 8) {
  const int qs = (g + 3) / 4;
  int w = 1;
  while (w * 2 * qs <= max_waves && hk % (w * 2) == 0) w *= 2;
  return w;
}
inline int balance_max_wgs(int hk, int g, int budget = kWaveBudget) {
  const int qs = (g + 3) / 4;
  const int n = budget / (hk * qs);
  return n < 1 ? 1 : n;
}

}  // namespace tqk
