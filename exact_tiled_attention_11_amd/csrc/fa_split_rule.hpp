// The split plan of the paged decode, shared by the host queries
// (fa_decode_max_splits, fa_decode_workspace_size, fa_decode_plan) and the
// kernels, so both always agree.
//
// "3.4 Attention Kernels", sections "Decode attention and Flash-Decoding",
// "Worked example" and "In practice": the keys of a sequence are cut into
// chunks so that enough workgroups stream the cache to keep every CU busy,
// the count following from the batch size, the head count and the context
// length. Here a sequence with v visible tokens gets ceil(v / C) chunks of
// about C tokens, at most K, where C and K depend on how many (sequence, KV
// head) pairs P the batch has:
//   * C = clamp(kChunkPerPair * P, kMinChunk, kMaxChunk): with few pairs
//     (batch 1 with 8 KV heads: 8 pairs) the chunks are short, so that long
//     sequences alone fill the GPU (a 32K context gives 32 chunks per KV
//     head, 256 workgroups); with many pairs (64 sequences x 8 KV heads:
//     2048 tokens) the pairs already fill the GPU and a split only adds a
//     workgroup's fixed costs (query load, page-id staging, final wave merge)
//     and a partial for the merge;
//   * K = ceil(kTargetChunks / P): with many pairs, long sequences are still
//     cut into a few chunks (8 at 64 x 8 pairs), so that no workgroup runs
//     far longer than the others and the launch ends without a long tail.
// The constants were chosen by measurement on the decode workloads: chunks of
// 1024 tokens at batch 1 and 8 (32 per 32K-token sequence); at batch 64,
// chunks of 2048 tokens and at most 8 per sequence (0.76 ms for the
// 1024..32768-token batch, against 0.80 ms for 4096-token chunks; 0.17 ms
// for the same batch with a 4096-token window).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

constexpr int kMinChunk = 1024;
constexpr int kMaxChunk = 4096;
constexpr int kChunkPerPair = 4;
// At most ceil(kTargetChunks / pairs) chunks per sequence: about
// kTargetChunks (sequence, KV head, chunk) workgroups when every sequence is
// long, sixteen per CU.
constexpr long long kTargetChunks = 4096;

// Tokens of a sequence of `len` cached tokens the query sees under a window
// of the newest `window` tokens (0: all); 0 for a length outside
// [0, max_len] (a contract violation, whose output is NaN anyway).
__host__ __device__ inline int visible_tokens(int len, int window, long long max_len) {
  if (len < 0 || len > max_len) return 0;
  return (window > 0 && len > window) ? window : len;
}

// Chunk length C for a batch of B sequences with Hkv KV heads each.
__host__ __device__ inline int decode_chunk_tokens(int B, int Hkv) {
  const long long c = static_cast<long long>(kChunkPerPair) * (B > 0 ? B : 1) * Hkv;
  return static_cast<int>(c < kMinChunk ? kMinChunk : c > kMaxChunk ? kMaxChunk : c);
}

// Partial slots per (sequence, head): the most chunks any sequence can get
// with at most max_pages pages of FA_PAGE_SIZE tokens; `fixed` > 0 forces it.
__host__ __device__ inline int decode_max_splits(int B, int Hkv, int max_pages, int window,
                                                 int fixed) {
  if (fixed > 0) return fixed;
  long long lmax = static_cast<long long>(max_pages) * FA_PAGE_SIZE;
  if (window > 0 && window < lmax) lmax = window;
  const int c = decode_chunk_tokens(B, Hkv);
  long long s = (lmax + c - 1) / c;
  const long long pairs = static_cast<long long>(B > 0 ? B : 1) * Hkv;
  const long long cap = (kTargetChunks + pairs - 1) / pairs;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  if (s > FA_MAX_SPLITS) s = FA_MAX_SPLITS;
  return static_cast<int>(s);
}

// Chunks of a sequence with `vis` visible tokens: ceil(vis / chunk) in
// [1, max_splits]; `fixed` > 0 forces that count.
__host__ __device__ inline int decode_splits(int vis, int chunk, int max_splits, int fixed) {
  if (fixed > 0) return fixed;
  long long s = (static_cast<long long>(vis) + chunk - 1) / chunk;
  if (s < 1) s = 1;
  if (s > max_splits) s = max_splits;
  return static_cast<int>(s);
}

// Chunk `split` of `nsplit` over `npages` pages: pages [begin, end), the
// near-equal page-aligned cut of numpy.array_split.
__host__ __device__ inline void split_pages(int npages, int nsplit, int split, int* begin,
                                            int* end) {
  const int q = npages / nsplit, r = npages % nsplit;
  *begin = split * q + (split < r ? split : r);
  *end = *begin + q + (split < r ? 1 : 0);
}

}  // namespace fa
