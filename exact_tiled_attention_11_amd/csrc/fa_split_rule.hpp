// The per-sequence split rule of the paged decode, shared by the host query
// (fa_decode_num_splits) and the kernels so both always agree.
#pragma once

#include <hip/hip_runtime.h>

#include "fa.h"

namespace fa {

// Smallest chunk (tokens) when the count is chosen automatically: sequences
// are cut into as many chunks of at least this many tokens as possible, up to
// FA_MAX_SPLITS. Many small chunks keep every CU streaming until the end of
// the launch even when sequence lengths differ by 30x.
constexpr int kSplitTokens = 256;

// Number of key chunks for a sequence of `len` tokens; `fixed` > 0 forces it.
__host__ __device__ inline int decode_splits(int len, int fixed) {
  if (fixed > 0) return fixed;
  int s = (len + kSplitTokens - 1) / kSplitTokens;
  if (s < 1) s = 1;
  if (s > FA_MAX_SPLITS) s = FA_MAX_SPLITS;
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
