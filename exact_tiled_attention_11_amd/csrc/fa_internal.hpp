// Internal launch interfaces between the C ABI layer (fa_api.hip) and the
// kernel translation units. Arguments reaching these functions have been
// validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

struct ForwardArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  fa_dtype in_dtype, out_dtype;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  int B, H, Hkv, d, page_size, max_pages, num_pages;
  float scale;
  int num_splits;  // 0 = per-sequence rule, else fixed
  int window;      // > 0: only the newest `window` keys are visible
  float softcap;   // > 0: scores x become softcap * tanh(x / softcap)
  fa_dtype dtype, out_dtype;
  float* part_o;    // [B, H, S, d] fp32
  float* part_lse;  // [B, H, S]    fp32
  int max_splits;   // S
};

struct ForwardPagedArgs {
  const void* q;             // [total_q, H, d]
  const int32_t* qo_indptr;  // [B + 1]
  const void* k_pool;        // [num_pages, 16, Hkv, d]
  const void* v_pool;
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* kv_lens;      // [B]
  void* o;                   // [total_q, H, d]
  float* lse;                // [total_q, H]
  int B, H, Hkv, d, total_q, max_q_len, max_pages, num_pages;
  float scale;
  int causal;
  fa_dtype dtype, out_dtype;
  // qo_indptr / kv_lens may be NULL: one sequence of all total_q rows /
  // fixed_kv_len keys per sequence.
  int fixed_kv_len = 0;
  // kv_splits > 1 (non-causal only): write fp32 partials instead of O, LSE.
  int kv_splits = 1;
  float* part_o = nullptr;    // [total_q * H, kv_splits, d]
  float* part_lse = nullptr;  // [total_q * H, kv_splits]
};

struct MergeArgs {
  const float* o_parts;
  const float* lse_parts;
  const int32_t* num_parts;  // may be NULL
  void* o;
  float* lse;
  int R, S, d;
  fa_dtype out_dtype;
  const float* o_extra = nullptr;    // optional extra part per row: [R, d]
  const float* lse_extra = nullptr;  // [R]
};

// Size of the library's own partial-result buffer (fa_decode_paged_noalloc).
constexpr size_t kDecodeScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
// Device address of that buffer on the current device (looked up once per
// device, then cached).
hipError_t decode_scratch(void** ptr);

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_paged(const ForwardPagedArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// The one-query sequences of a ragged batch (qo_indptr[b + 1] - qo_indptr[b]
// == 1) through the decode kernel, one workgroup per (sequence, KV head);
// needs qo_indptr and kv_lens, H / Hkv <= 16, no partial mode.
hipError_t launch_decode_rows(const ForwardPagedArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

}  // namespace fa
