// The per-sequence split plan of the paged decode, shared by the host queries
// (fa_decode_max_splits, fa_decode_num_splits, fa_decode_workspace_size) and
// the kernels, so both always agree.
//
// "3.4 Attention Kernels", sections "Decode attention and Flash-Decoding",
// "Worked example" and "In practice": the keys of a sequence are cut into
// chunks so that enough workgroups stream the cache to keep every CU busy,
// and the count follows from the batch size, the head count and the context
// length. Here:
//   * a chunk holds at least kSplitTokens tokens, so short sequences stay in
//     one piece and no chunk is dominated by its fixed costs;
//   * the most chunks a sequence gets is a cap that depends on how many
//     (sequence, KV head) units the batch already has: about kTargetUnits
//     workgroups in all (16 per CU), between 1 and FA_MAX_SPLITS chunks. At
//     batch 1 with 8 KV heads that is 64 chunks (512 workgroups, two per CU
//     at once); at 64 sequences 16; at 256 sequences 4.
#pragma once

#include <hip/hip_runtime.h>

#include "fa.h"

namespace fa {

constexpr int kSplitTokens = 256;
constexpr int kTargetUnits = 8192;

// Chunk cap for a batch of B sequences with Hkv KV heads each; `fixed` > 0
// forces that count. Also the number of partial slots per (sequence, head)
// in the workspace.
__host__ __device__ inline int decode_max_splits(int B, int Hkv, int fixed) {
  if (fixed > 0) return fixed;
  const long long units = static_cast<long long>(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
  long long cap = (kTargetUnits + units - 1) / units;
  if (cap < 1) cap = 1;
  if (cap > FA_MAX_SPLITS) cap = FA_MAX_SPLITS;
  return static_cast<int>(cap);
}

// Number of key chunks for a sequence of `len` visible tokens under the cap
// `max_splits` (from decode_max_splits); `fixed` > 0 forces that count.
__host__ __device__ inline int decode_splits(int len, int max_splits, int fixed) {
  if (fixed > 0) return fixed;
  int s = (len + kSplitTokens - 1) / kSplitTokens;
  if (s < 1) s = 1;
  if (s > max_splits) s = max_splits;
  return s;
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
