// Stream-K tile location shared by the persistent decode kernels: the
// tiles of a batch are its sequences' blocks in (sequence, block) order, one
// tile per BS-token block; a wave finds the sequence and block of its first
// tile by scanning seq_lens.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_wave.h"

namespace pa {

template <int BS>
__device__ __forceinline__ int blocks_of(int L) { return (L + BS - 1) / BS; }

// Block counts of sequences c0 + 64*j + lane, j < K: the loads are
// unconditional (index clamped, count masked) so all K are in flight together
// and a scan over seq_lens waits one memory latency per 64*K sequences.
template <int BS, int K>
__device__ __forceinline__ void block_counts(const DecodeArgs& a, int c0, int lane, int (&nb)[K]) {
  const int S = a.num_seqs;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int s = c0 + 64 * j + lane;
    const int L = a.seq_lens[min(s, S - 1)];
    nb[j] = blocks_of<BS>(clamp_len(L, a.max_seq_len)) & -(int)(s < S);
  }
}

// Total blocks over all sequences.
template <int BS, int K>
__device__ __forceinline__ int total_blocks(const DecodeArgs& a, int lane) {
  int T = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64 * K) {
    int nb[K];
    block_counts<BS, K>(a, c0, lane, nb);
#pragma unroll
    for (int j = 0; j < K; ++j) T += wave_sum(nb[j]);
  }
  return T;
}

// The sequence whose block range (in sequence order, counted from sequence
// c_begin) holds block r, and the block's index within it.
template <int BS, int K>
__device__ __forceinline__ void find_block(const DecodeArgs& a, int lane, int r, int& seq, int& blk, int c_begin = 0) {
  int running = 0;
  for (int c0 = c_begin; c0 < a.num_seqs; c0 += 64 * K) {
    int nb[K];
    block_counts<BS, K>(a, c0, lane, nb);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int incl = wave_incl_scan(nb[j], lane) + running;
      const int excl = incl - nb[j];
      const uint64_t hit = __builtin_amdgcn_ballot_w64(nb[j] > 0 && excl <= r && r < incl);
      if (hit) {
        const int ln = __builtin_ctzll(hit);
        seq = c0 + 64 * j + ln;
        blk = r - __builtin_amdgcn_readlane(excl, ln);
        return;
      }
      running = __builtin_amdgcn_readlane(incl, 63);
    }
  }
}

// Total blocks T of the batch. Up to 128 sequences: one two-chunk batch.
// More: batches of 16 chunks (1024 sequences), whose block totals lane b of
// bsum keeps for batch b, so locate_block scans only the batch that holds a
// wave's first tile.
constexpr int kScanBig = 16;

template <int BS>
__device__ __forceinline__ int count_blocks(const DecodeArgs& a, int lane, int& bsum) {
  bsum = 0;
  if (a.num_seqs <= 128) return total_blocks<BS, 2>(a, lane);
  int T = 0;
  for (int c0 = 0, b = 0; c0 < a.num_seqs; c0 += 64 * kScanBig, ++b) {
    int nb[kScanBig];
    block_counts<BS, kScanBig>(a, c0, lane, nb);
    int t = 0;
#pragma unroll
    for (int j = 0; j < kScanBig; ++j) t += nb[j];
    const int bt = wave_sum(t);
    if (lane == b) bsum = bt;
    T += bt;
  }
  return T;
}

// Sequence and block of tile r (0 <= r < T), with bsum from count_blocks.
template <int BS>
__device__ __forceinline__ void locate_block(const DecodeArgs& a, int lane, int r, int bsum, int& seq, int& blk) {
  if (a.num_seqs <= 128) {
    find_block<BS, 2>(a, lane, r, seq, blk);
  } else if (a.num_seqs <= 64 * 64 * kScanBig) {
    const int incl = wave_incl_scan(bsum, lane);
    const int excl = incl - bsum;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(bsum > 0 && excl <= r && r < incl);
    const int b = hit ? __builtin_ctzll(hit) : 0;
    find_block<BS, kScanBig>(a, lane, r - __builtin_amdgcn_readlane(excl, b), seq, blk, 64 * kScanBig * b);
  } else {
    find_block<BS, kScanBig>(a, lane, r, seq, blk);
  }
}

}  // namespace pa
