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

// Sequence length b clamped to [0, block-table capacity].
__device__ __forceinline__ int clamped_seq(const DecodeParams& p, int b) {
  int64_t s64 = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  s64 = s64 < 0 ? 0 : (s64 > cap ? cap : s64);
  return (int)s64;
}

// Split geometry of a sequence of `seq` tokens (already clamped).
__device__ __forceinline__ SeqSplits splits_of(const DecodeParams& p, int seq) {
  SeqSplits r;
  r.seq = seq;
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

__device__ __forceinline__ SeqSplits seq_splits(const DecodeParams& p, int b) {
  return splits_of(p, clamped_seq(p, b));
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

// LDS the stage-1 prologue needs: prefix[B + 1] followed by seql[B].
inline size_t balance_lds_bytes(int B) { return (size_t)(2 * B + 1) * sizeof(int); }

// Prologue of the balanced stage 1, run by all NT threads of a workgroup:
// the clamped sequence lengths into seql[0, B), the exclusive prefix sums of
// their tile counts into prefix[0, B] (workgroup 0 also publishes them to
// wsx for stage 2). `scan` holds NT / 64 ints. Returns N, the total tile
// count. Ends with a barrier.
template <int NT>
__device__ __forceinline__ int balance_prologue(const DecodeParams& p, int* prefix, int* seql,
                                                int* scan) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (p.B + NT - 1) / NT;  // consecutive sequences per thread
  int run = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) {
      const int sq = clamped_seq(p, b);
      seql[b] = sq;
      run += seq_tiles(splits_of(p, sq));
      prefix[b + 1] = run;
    }
  }
  // inclusive scan of the per-thread sums: across the wave, then waves
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  int N = 0, before = 0;
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; ++w2) {
    const int t = scan[w2];
    N += t;
    before += w2 < wave ? t : 0;
  }
  const int excl = before + incl - run;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) {
      prefix[b + 1] += excl;
      if (blockIdx.x == 0) p.wsx[b + 1] = prefix[b + 1];
    }
  }
  if (tid == 0) {
    prefix[0] = 0;
    if (blockIdx.x == 0) p.wsx[0] = 0;
  }
  __syncthreads();
  return N;
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
