// The extern "C" entry points of include/fa.h: argument validation on the
// host, then launches on the caller's stream. Nothing here allocates or keeps
// state; every check runs before the first HIP call so an invalid call has
// no side effect at all.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>

#include "fa.h"
#include "fa_internal.hpp"
#include "fa_split_rule.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;

// HIP limits the threads of a launch along x (workgroups x workgroup size)
// to 2^32 - 1.
constexpr int64_t kMaxThreadsX = (int64_t{1} << 32) - 1;
constexpr int64_t kFwd16Threads = 512;   // 8 waves
constexpr int64_t kFwd32Threads = 256;   // 4 waves
constexpr int64_t kMergeRowsPerBlock = 4, kMergeThreads = 256;
constexpr int64_t kDecodeThreads = 256;  // 4 waves
bool grid_fits(int64_t workgroups, int64_t threads) {
  return workgroups >= 0 && workgroups <= kMaxThreadsX / threads;
}
// Launch size of the merge kernel for R rows.
bool merge_fits(int64_t rows) {
  return grid_fits((rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock, kMergeThreads);
}

bool valid_dtype(fa_dtype t) { return t == FA_F32 || t == FA_F16 || t == FA_BF16; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Workgroups of a 16-bit forward launch: (batch, KV head) groups padded to a
// multiple of the 8 XCDs, times the work units per group (blocks of 256
// packed (query, head) rows; causal pairs two blocks per unit).
int64_t forward16_grid(int64_t B, int64_t Hkv, int64_t group, int64_t max_q, bool causal) {
  const int64_t blocks = (max_q * group + 255) / 256;
  const int64_t units = causal ? (blocks + 1) / 2 : blocks;
  return (B * Hkv + 7) / 8 * 8 * units;
}

// The kernels move data in 16-byte vectors.
// 16-byte aligned and inside the 48-bit GPU virtual address space (the base
// field of a buffer resource holds address bits 0..47 and nothing above).
bool aligned16(const void* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return (a & 15u) == 0 && (static_cast<uint64_t>(a) >> 48) == 0;
}

// Query heads per KV head the decode kernels serve together (head slots of
// their matrix-core tiles).
constexpr int kMaxDecodeGroup = 16;

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: a size is negative, inconsistent or too large";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but not implemented for these sizes or types";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or smaller than required";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch failure";
    case FA_ERR_BAD_ARG: return "FA_ERR_BAD_ARG: an argument is out of range";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the sizes need more partial-result memory than the library's "
             "fixed scratch buffer holds (use the entry point with a caller workspace)";
  }
  return "unknown fa_status";
}

const char* fa_version(void) { return "0.1.0"; }

fa_status fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                     int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     fa_dtype in_dtype, fa_dtype out_dtype, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return FA_ERR_BAD_SHAPE;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return FA_ERR_BAD_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_ARG;
  if (!scale_ok(scale)) return FA_ERR_BAD_ARG;
  if (!head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (out_dtype != in_dtype && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  const int64_t q_elems = int64_t{B} * Nq * H * d;
  const int64_t kv_elems = int64_t{B} * Nk * Hkv * d;
  const bool grid_ok =
      in_dtype == FA_F32
          ? grid_fits(int64_t{B} * H * ((int64_t{Nq} + 127) / 128), kFwd32Threads)
          : grid_fits(forward16_grid(B, Hkv, H / Hkv, Nq, causal != 0), kFwd16Threads);
  if (q_elems > kMaxElems || kv_elems > kMaxElems || !grid_ok) return FA_ERR_BAD_SHAPE;
  if (B == 0 || Nq == 0) return FA_OK;
  if (!Q || !O || !LSE || (Nk > 0 && (!K || !V))) return FA_ERR_NULL_PTR;
  if (!aligned16(Q) || !aligned16(O) || (Nk > 0 && (!aligned16(K) || !aligned16(V))))
    return FA_ERR_BAD_ARG;
  fa::ForwardArgs a{Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal, in_dtype, out_dtype};
  return from_hip(fa::launch_forward(a, static_cast<hipStream_t>(stream)));
}

fa_status fa_forward_paged(const void* Q, const int32_t* qo_indptr, const void* K_pool,
                           const void* V_pool, const int32_t* block_table, const int32_t* kv_lens,
                           void* O, float* LSE, int B, int H, int Hkv, int d, int total_q,
                           int max_q_len, int page_size, int max_pages_per_seq, int num_pages,
                           float scale, int causal, fa_dtype dtype, fa_dtype out_dtype,
                           void* stream) {
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || total_q < 0 || max_q_len < 0 ||
      max_pages_per_seq < 1 || num_pages < 1 || page_size < 1)
    return FA_ERR_BAD_SHAPE;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return FA_ERR_BAD_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_ARG;
  if (!scale_ok(scale)) return FA_ERR_BAD_ARG;
  if (!head_dim_ok(d) || page_size != FA_PAGE_SIZE || dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (out_dtype != dtype && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (int64_t{total_q} * H * d > kMaxElems ||
      int64_t{num_pages} * page_size * Hkv * d > kMaxElems ||
      int64_t{B} * max_pages_per_seq > kMaxElems ||
      int64_t{max_pages_per_seq} * page_size > kMaxElems ||
      !grid_fits(forward16_grid(B, Hkv, H / Hkv, max_q_len, causal != 0), kFwd16Threads))
    return FA_ERR_BAD_SHAPE;
  if (B == 0 || total_q == 0 || max_q_len == 0) return FA_OK;
  if (!Q || !qo_indptr || !K_pool || !V_pool || !block_table || !kv_lens || !O || !LSE)
    return FA_ERR_NULL_PTR;
  if (!aligned16(Q) || !aligned16(O) || !aligned16(K_pool) || !aligned16(V_pool))
    return FA_ERR_BAD_ARG;
  fa::ForwardPagedArgs a{Q, qo_indptr, K_pool, V_pool, block_table, kv_lens, O, LSE,
                         B, H, Hkv, d, total_q, max_q_len, max_pages_per_seq, num_pages,
                         scale, causal, dtype, out_dtype};
  return from_hip(fa::launch_forward_paged(a, static_cast<hipStream_t>(stream)));
}

int fa_cascade_num_splits(int prefix_len, int total_q, int H, int Hkv, int prefix_splits) {
  if (prefix_len < 0 || total_q < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || prefix_splits < 0 ||
      prefix_splits > FA_CASCADE_MAX_SPLITS)
    return -1;
  if (prefix_splits > 0) return prefix_splits;
  // Enough workgroups for two per CU, but at least 512 prefix keys per split.
  const int64_t blocks = std::max<int64_t>(1, (int64_t{total_q} * (H / Hkv) + 255) / 256);
  const int64_t want = (512 + int64_t{Hkv} * blocks - 1) / (int64_t{Hkv} * blocks);
  const int64_t cap = (int64_t{prefix_len} + 511) / 512;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({want, cap,
                                                                  FA_CASCADE_MAX_SPLITS})));
}

size_t fa_cascade_workspace_size(int total_q, int H, int d, int num_splits) {
  if (total_q < 0 || H < 1 || d < 1 || num_splits < 1 || num_splits > FA_CASCADE_MAX_SPLITS)
    return 0;
  const size_t rows = static_cast<size_t>(total_q) * H;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al(rows * num_splits * d * 4) + al(rows * num_splits * 4) + al(rows * d * 4) + rows * 4;
}

fa_status fa_cascade(const void* Q, const int32_t* qo_indptr, const void* K_pool,
                     const void* V_pool, const int32_t* prefix_pages, int prefix_len,
                     int prefix_splits, const int32_t* block_table, const int32_t* kv_lens,
                     void* O, float* LSE, int B, int H, int Hkv, int d, int total_q,
                     int max_q_len, int page_size, int max_pages_per_seq, int num_pages,
                     float scale, int causal, fa_dtype dtype, fa_dtype out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  // The suffix pass is exactly fa_forward_paged; validate it first (it
  // launches nothing on error).
  if (prefix_len < 0 || prefix_splits < 0 || prefix_splits > FA_CASCADE_MAX_SPLITS)
    return FA_ERR_BAD_ARG;
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || total_q < 0 || max_q_len < 0 ||
      max_pages_per_seq < 1 || num_pages < 1 || page_size < 1)
    return FA_ERR_BAD_SHAPE;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return FA_ERR_BAD_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_BAD_ARG;
  if (!scale_ok(scale)) return FA_ERR_BAD_ARG;
  if (!head_dim_ok(d) || page_size != FA_PAGE_SIZE || dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (out_dtype != dtype && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  const int S = fa_cascade_num_splits(prefix_len, total_q, H, Hkv, prefix_splits);
  const int64_t prefix_pages_n = (int64_t{prefix_len} + page_size - 1) / page_size;
  if (int64_t{total_q} * H * d > kMaxElems || int64_t{total_q} * H * S * d > kMaxElems ||
      int64_t{num_pages} * page_size * Hkv * d > kMaxElems ||
      int64_t{B} * max_pages_per_seq > kMaxElems ||
      int64_t{max_pages_per_seq} * page_size > kMaxElems ||
      !grid_fits(forward16_grid(B, Hkv, H / Hkv, max_q_len, causal != 0), kFwd16Threads) ||
      !grid_fits(forward16_grid(1, Hkv, H / Hkv, total_q, false) * S, kFwd16Threads) ||
      !merge_fits(int64_t{total_q} * H))
    return FA_ERR_BAD_SHAPE;
  if (total_q == 0) return FA_OK;
  if (!Q || !K_pool || !V_pool || !O || !LSE || (prefix_len > 0 && !prefix_pages) ||
      (B > 0 && (!qo_indptr || !block_table || !kv_lens)))
    return FA_ERR_NULL_PTR;
  if (!aligned16(Q) || !aligned16(O) || !aligned16(K_pool) || !aligned16(V_pool))
    return FA_ERR_BAD_ARG;
  const size_t need = fa_cascade_workspace_size(total_q, H, d, S);
  if (prefix_len > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);

  fa::ForwardPagedArgs suf{Q, qo_indptr, K_pool, V_pool, block_table, kv_lens, O, LSE,
                           B, H, Hkv, d, total_q, max_q_len, max_pages_per_seq, num_pages,
                           scale, causal, dtype, out_dtype};
  if (prefix_len == 0) {   // nothing shared: the suffix pass is the answer
    if (B == 0 || max_q_len == 0) return FA_OK;
    return from_hip(fa::launch_forward_paged(suf, st));
  }
  const size_t rows = static_cast<size_t>(total_q) * H;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(w);
  float* part_lse = reinterpret_cast<float*>(w + al(rows * S * d * 4));
  float* suf_o = reinterpret_cast<float*>(w + al(rows * S * d * 4) + al(rows * S * 4));
  float* suf_lse = reinterpret_cast<float*>(w + al(rows * S * d * 4) + al(rows * S * 4) +
                                            al(rows * d * 4));
  // 1. Shared prefix: all query rows against the prefix pages, non-causal,
  //    split over S key ranges, fp32 partials.
  fa::ForwardPagedArgs pre{Q, nullptr, K_pool, V_pool, prefix_pages, nullptr, nullptr, nullptr,
                           1, H, Hkv, d, total_q, total_q,
                           static_cast<int>(prefix_pages_n), num_pages, scale, 0, dtype,
                           FA_F32};
  pre.fixed_kv_len = prefix_len;
  pre.kv_splits = S;
  pre.part_o = part_o;
  pre.part_lse = part_lse;
  hipError_t e = fa::launch_forward_paged(pre, st);
  if (e != hipSuccess) return FA_ERR_HIP;
  // 2. Each sequence's own suffix, fp32.
  suf.o = suf_o;
  suf.lse = suf_lse;
  suf.out_dtype = FA_F32;
  if (B > 0 && max_q_len > 0) {
    e = fa::launch_forward_paged(suf, st);
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  // 3. Merge the S prefix parts and the suffix part of every (row, head).
  fa::MergeArgs m{part_o, part_lse, nullptr, O, LSE, static_cast<int>(rows), S, d, out_dtype};
  if (B > 0 && max_q_len > 0) {
    m.o_extra = suf_o;
    m.lse_extra = suf_lse;
  }
  return from_hip(fa::launch_merge(m, st));
}

int fa_decode_max_splits(int B, int Hkv, int max_pages_per_seq, int window, int num_splits) {
  if (B < 0 || Hkv < 1 || max_pages_per_seq < 1 || window < 0 || num_splits < 0 ||
      num_splits > FA_MAX_SPLITS)
    return -1;
  return fa::decode_max_splits(B, Hkv, max_pages_per_seq, window, num_splits);
}

size_t fa_decode_workspace_size(int B, int H, int Hkv, int d, int max_pages_per_seq, int window,
                                int num_splits) {
  const int S = fa_decode_max_splits(B, Hkv, max_pages_per_seq, window, num_splits);
  if (H < 1 || H % Hkv != 0 || d < 1 || S < 1) return 0;
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(H) * S;
  const size_t o_bytes = (rows * static_cast<size_t>(d) * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * sizeof(float);
}

fa_status fa_decode_plan(const int32_t* seq_lens_host, int B, int Hkv, int max_pages_per_seq,
                         int window, int num_splits, int32_t* splits_out) {
  if (B < 0 || Hkv < 1 || max_pages_per_seq < 1) return FA_ERR_BAD_SHAPE;
  if (window < 0 || num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_BAD_ARG;
  if (B > 0 && (!seq_lens_host || !splits_out)) return FA_ERR_NULL_PTR;
  const int S = fa::decode_max_splits(B, Hkv, max_pages_per_seq, window, num_splits);
  const int C = fa::decode_chunk_tokens(B, Hkv);
  const long long max_len = static_cast<long long>(max_pages_per_seq) * FA_PAGE_SIZE;
  for (int b = 0; b < B; ++b)
    splits_out[b] =
        fa::decode_splits(fa::visible_tokens(seq_lens_host[b], window, max_len), C, S, num_splits);
  return FA_OK;
}

}  // extern "C"

namespace {

// The partial (o, lse) slots of a decode in `workspace`: o [B, H, S, d] fp32,
// then lse [B, H, S] fp32 at the next 256-byte boundary.
void set_partials(fa::DecodeArgs* a, void* workspace) {
  const size_t rows = static_cast<size_t>(a->B) * a->H * a->max_splits;
  char* w = static_cast<char*>(workspace);
  a->part_o = reinterpret_cast<float*>(w);
  a->part_lse =
      w ? reinterpret_cast<float*>(w + (rows * a->d * sizeof(float) + 255) / 256 * 256) : nullptr;
}

// Validates a decode call and fills `a`; launches nothing. `*empty` is set
// when the call is valid but has no work (B == 0).
fa_status decode_prepare(const void* q, const void* K_pool, const void* V_pool,
                         const int32_t* block_table, const int32_t* seq_lens, void* O, float* LSE,
                         int B, int H, int Hkv, int d, int page_size, int max_pages_per_seq,
                         int num_pages, float scale, int num_splits, int window, float softcap,
                         fa_dtype dtype, fa_dtype out_dtype, void* workspace,
                         size_t workspace_bytes, fa::DecodeArgs* out, bool* empty,
                         bool check_workspace = true) {
  *empty = false;
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1 ||
      page_size < 1)
    return FA_ERR_BAD_SHAPE;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_BAD_ARG;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return FA_ERR_BAD_ARG;
  if (!scale_ok(scale)) return FA_ERR_BAD_ARG;
  if (window < 0 || !std::isfinite(softcap) || softcap < 0.f) return FA_ERR_BAD_ARG;
  const int G = H / Hkv;
  if (!head_dim_ok(d) || page_size != FA_PAGE_SIZE || dtype == FA_F32 || G > kMaxDecodeGroup)
    return FA_ERR_UNSUPPORTED;
  if (out_dtype != dtype && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (int64_t{num_pages} * page_size * Hkv * d > kMaxElems ||
      int64_t{B} * max_pages_per_seq > kMaxElems || int64_t{B} * H * d > kMaxElems ||
      int64_t{max_pages_per_seq} * page_size > kMaxElems || B > 65535 || Hkv > 65535 ||
      !merge_fits(int64_t{B} * H) ||
      !grid_fits(int64_t{B} * Hkv *
                     fa::decode_max_splits(B, Hkv, max_pages_per_seq, window, num_splits),
                 kDecodeThreads))
    return FA_ERR_BAD_SHAPE;
  if (B == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !K_pool || !V_pool || !block_table || !seq_lens || !O || !LSE)
    return FA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(K_pool) || !aligned16(V_pool)) return FA_ERR_BAD_ARG;
  const int S = fa::decode_max_splits(B, Hkv, max_pages_per_seq, window, num_splits);
  const size_t need =
      fa_decode_workspace_size(B, H, Hkv, d, max_pages_per_seq, window, num_splits);
  if (check_workspace && S > 1 && (workspace == nullptr || workspace_bytes < need))
    return FA_ERR_WORKSPACE;
  if (check_workspace && S > 1 && !aligned16(workspace)) return FA_ERR_BAD_ARG;
  fa::DecodeArgs a;
  a.q = q; a.k_pool = K_pool; a.v_pool = V_pool;
  a.block_table = block_table; a.seq_lens = seq_lens;
  a.o = O; a.lse = LSE;
  a.B = B; a.H = H; a.Hkv = Hkv; a.d = d; a.page_size = page_size;
  a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  a.scale = scale; a.num_splits = num_splits;
  a.window = window; a.softcap = softcap;
  a.dtype = dtype; a.out_dtype = out_dtype;
  a.max_splits = S;
  set_partials(&a, workspace);
  *out = a;
  return FA_OK;
}

fa_status decode_impl(const void* q, const void* K_pool, const void* V_pool,
                      const int32_t* block_table, const int32_t* seq_lens, void* O, float* LSE,
                      int B, int H, int Hkv, int d, int page_size, int max_pages_per_seq,
                      int num_pages, float scale, int num_splits, int window, float softcap,
                      fa_dtype dtype, fa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  fa::DecodeArgs a;
  bool empty;
  const fa_status st = decode_prepare(q, K_pool, V_pool, block_table, seq_lens, O, LSE, B, H,
                                      Hkv, d, page_size, max_pages_per_seq, num_pages, scale,
                                      num_splits, window, softcap, dtype, out_dtype, workspace,
                                      workspace_bytes, &a, &empty);
  if (st != FA_OK || empty) return st;
  return from_hip(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

fa_status fa_decode_paged(const void* q, const void* K_pool, const void* V_pool,
                          const int32_t* block_table, const int32_t* seq_lens, void* O, float* LSE,
                          int B, int H, int Hkv, int d, int page_size, int max_pages_per_seq,
                          int num_pages, float scale, int num_splits, fa_dtype dtype,
                          fa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_impl(q, K_pool, V_pool, block_table, seq_lens, O, LSE, B, H, Hkv, d, page_size,
                     max_pages_per_seq, num_pages, scale, num_splits, 0, 0.f, dtype, out_dtype,
                     workspace, workspace_bytes, stream);
}

fa_status fa_decode_paged_ex(const void* q, const void* K_pool, const void* V_pool,
                             const int32_t* block_table, const int32_t* seq_lens, void* O,
                             float* LSE, int B, int H, int Hkv, int d, int page_size,
                             int max_pages_per_seq, int num_pages, float scale, int num_splits,
                             int window, float softcap, fa_dtype dtype, fa_dtype out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, K_pool, V_pool, block_table, seq_lens, O, LSE, B, H, Hkv, d, page_size,
                     max_pages_per_seq, num_pages, scale, num_splits, window, softcap, dtype,
                     out_dtype, workspace, workspace_bytes, stream);
}

fa_status fa_decode_paged_noalloc(const void* q, const void* K_pool, const void* V_pool,
                                  const int32_t* block_table, const int32_t* seq_lens, void* O,
                                  float* LSE, int B, int H, int Hkv, int d, int page_size,
                                  int max_pages_per_seq, int num_pages, float scale,
                                  int num_splits, int window, float softcap, fa_dtype dtype,
                                  fa_dtype out_dtype, void* stream) {
  // Everything but the workspace is validated exactly as for
  // fa_decode_paged_ex; the partials then go to the library's fixed buffer.
  fa::DecodeArgs a;
  bool empty;
  fa_status st = decode_prepare(q, K_pool, V_pool, block_table, seq_lens, O, LSE, B, H, Hkv, d,
                                page_size, max_pages_per_seq, num_pages, scale, num_splits,
                                window, softcap, dtype, out_dtype, nullptr, 0, &a, &empty,
                                /*check_workspace=*/false);
  if (st != FA_OK || empty) return st;
  if (fa_decode_workspace_size(B, H, Hkv, d, max_pages_per_seq, window, num_splits) >
      fa::kDecodeScratchBytes)
    return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  set_partials(&a, ws);
  return from_hip(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

struct fa_decode_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

fa_status fa_decode_graph_create(fa_decode_graph** out, const void* q, const void* K_pool,
                                 const void* V_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, void* O, float* LSE, int B, int H,
                                 int Hkv, int d, int page_size, int max_pages_per_seq,
                                 int num_pages, float scale, int num_splits, int window,
                                 float softcap, fa_dtype dtype, fa_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes) {
  if (!out) return FA_ERR_NULL_PTR;
  *out = nullptr;
  fa::DecodeArgs a;
  bool empty;
  const fa_status st = decode_prepare(q, K_pool, V_pool, block_table, seq_lens, O, LSE, B, H,
                                      Hkv, d, page_size, max_pages_per_seq, num_pages, scale,
                                      num_splits, window, softcap, dtype, out_dtype, workspace,
                                      workspace_bytes, &a, &empty);
  if (st != FA_OK) return st;
  hipStream_t cs;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return FA_ERR_HIP;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool ok = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) == hipSuccess;
  if (ok) {
    const hipError_t le = empty ? hipSuccess : fa::launch_decode(a, cs);
    const hipError_t ce = hipStreamEndCapture(cs, &graph);
    ok = le == hipSuccess && ce == hipSuccess && graph != nullptr;
  }
  if (ok) ok = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
  (void)hipStreamDestroy(cs);
  if (!ok) {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    return FA_ERR_HIP;
  }
  fa_decode_graph* g = new (std::nothrow) fa_decode_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return FA_ERR_HIP;
  }
  *out = g;
  return FA_OK;
}

fa_status fa_decode_graph_launch(const fa_decode_graph* g, void* stream) {
  if (!g) return FA_ERR_NULL_PTR;
  return from_hip(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

void fa_decode_graph_destroy(fa_decode_graph* g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

fa_status fa_merge_partials(const float* o_parts, const float* lse_parts, const int32_t* num_parts,
                            void* O, float* LSE, int R, int S, int d, fa_dtype out_dtype,
                            void* stream) {
  if (R < 0 || S < 1 || S > 1024 || d < 1 || d > 1024) return FA_ERR_BAD_SHAPE;
  if (!valid_dtype(out_dtype)) return FA_ERR_BAD_ARG;
  if (int64_t{R} * S * d > kMaxElems || !merge_fits(R)) return FA_ERR_BAD_SHAPE;
  if (R == 0) return FA_OK;
  if (!o_parts || !lse_parts || !O || !LSE) return FA_ERR_NULL_PTR;
  fa::MergeArgs a{o_parts, lse_parts, num_parts, O, LSE, R, S, d, out_dtype};
  return from_hip(fa::launch_merge(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
