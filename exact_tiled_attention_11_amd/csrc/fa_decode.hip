// Split-KV decode over a paged KV cache, and the merge of partial results.
//
// "3.4 Attention Kernels", section "Decode attention and Flash-Decoding":
// one query per sequence and head; the cached keys of a sequence are cut into
// chunks, each chunk's partial (m, l, acc) is computed by its own workgroup,
// and a small reduction kernel merges them with the merge rule of section
// "Online softmax". All query heads that share one KV head (the GQA group) are
// scored against each loaded key, so every K/V byte read from HBM is used G
// times. Pages are found through the block table ("Paged and ragged layouts:
// FlashInfer").
//
// Decode kernel, one workgroup (4 waves) per (sequence, KV head, chunk):
//   * wave w streams pages w, w+4, ... of the chunk; the next page's K and V
//     are loaded while the current one is processed;
//   * scores: S^T (16 tokens x 16 head slots) = K_page Q^T on a 16x16x32
//     matrix-core op, K loaded straight from HBM into the operand registers
//     (each lane 16 bytes of one token row); lane l then holds head l % 16
//     for tokens 4(l/16)..4(l/16)+3, only the first G head slots are real;
//   * online softmax per head with two cross-row exchanges (l^16, l^32);
//   * P V on the vector ALUs: the page's probabilities and rescale factors
//     go through a small per-wave LDS buffer to lanes that own 8 contiguous
//     d of a few token rows, V read with 16-byte coalesced loads;
//   * at the end the 4 wave states are merged in LDS with the same rule and
//     the chunk's (o, lse) is written: as the final output when the sequence
//     has one chunk, else as a partial for the merge kernel.
// Merge kernel, one wave per (sequence, head): M = max lse, weights e^(lse-M),
// fixed summation order, no atomics.
#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_split_rule.hpp"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kPage = FA_PAGE_SIZE;   // 16 token slots per page

struct DecParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* part_o;
  float* part_lse;
  int B, H, Hkv, max_pages, num_pages, num_splits, max_splits;
  float c;   // scale * log2(e)
};

__device__ __forceinline__ float nanf_() { return __builtin_nanf(""); }

template <class E, typename OutT, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecParams a) {
  constexpr int LPR = D / 8;           // lanes per token row in the P V layout
  constexpr int RPI = 64 / LPR;        // token rows covered per 16-byte load instruction
  constexpr int TPL = kPage / RPI;     // token rows per lane per page
  constexpr int NC = D / 32;           // 16x16x32 steps over d
  static_assert(G >= 1 && G <= 16, "head group must fit the 16 head slots");

  __shared__ float pbuf[kDecWaves][G][kPage];   // per-wave probabilities [head][token]
  __shared__ float abuf[kDecWaves][G];          // per-wave rescale factors
  __shared__ float wm[kDecWaves][G], wl[kDecWaves][G];
  __shared__ float wacc[kDecWaves][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int len = a.seq_lens[b];
  const bool bad_len = len < 0 || len > a.max_pages * kPage;
  const int nsplit = decode_splits(bad_len ? 0 : len, a.num_splits);
  if (split >= nsplit) return;                 // whole workgroup: uniform
  const int npages = bad_len ? 0 : (len + kPage - 1) / kPage;
  int pb, pe;
  split_pages(npages, nsplit, split, &pb, &pe);

  const int64_t row_stride = static_cast<int64_t>(a.Hkv) * D;   // between token slots
  const int64_t page_stride = row_stride * kPage;
  const uint16_t* kbase = a.k_pool + static_cast<int64_t>(hk) * D;
  const uint16_t* vbase = a.v_pool + static_cast<int64_t>(hk) * D;
  const int32_t* table = a.block_table + static_cast<int64_t>(b) * a.max_pages;

  // Q^T operand: lane l holds q[b, hk*G + l%16, 32c + 8(l/16) + j] (zero for
  // head slots >= G).
  const int hs = lane & 15, grp = lane >> 4;
  typename E::vec8 qop[NC];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.H + hk * G + hs) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (hs < G) u = *reinterpret_cast<const uint4*>(qrow + 32 * c);
      qop[c] = __builtin_bit_cast(typename E::vec8, u);
    }
  }

  // P V layout: lane owns d = 8e..8e+7 of token rows r*TPL .. r*TPL+TPL-1.
  const int e = lane % LPR, r = lane / LPR;

  float acc[G][8];
#pragma unroll
  for (int n = 0; n < G; ++n)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[n][j] = 0.f;
  float m_run = kNegInf, m2_run = kNegInf, l_run = 0.f;   // head slot hs
  bool bad_page = false;

  uint4 kc[NC], vc[TPL], kn[NC], vn[TPL];
  auto load_page = [&](int pg, uint4* kd, uint4* vd) {
    const uint16_t* kp = kbase + static_cast<int64_t>(pg) * page_stride;
    const uint16_t* vp = vbase + static_cast<int64_t>(pg) * page_stride;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kd[c] = *reinterpret_cast<const uint4*>(kp + hs * row_stride + 32 * c + 8 * grp);
#pragma unroll
    for (int i = 0; i < TPL; ++i)
      vd[i] = *reinterpret_cast<const uint4*>(vp + (r * TPL + i) * row_stride + 8 * e);
  };

  const int my_first = pb + wave;
  const int my_count = my_first < pe ? (pe - my_first + kDecWaves - 1) / kDecWaves : 0;

  // Page ids of this wave, 64 at a time, one per lane; read back with readlane.
  int ids = 0;
  auto fetch_ids = [&](int k0) {
    const int kk = k0 + lane;
    int v = 0;
    if (kk < my_count) v = table[my_first + kk * kDecWaves];
    ids = v;
  };
  auto page_id = [&](int k) -> int {
    int v = __builtin_amdgcn_readlane(ids, k & 63);
    if (v < 0 || v >= a.num_pages) {   // outside the pool: never dereferenced
      bad_page = true;
      v = 0;
    }
    return v;
  };

  if (my_count > 0) {
    fetch_ids(0);
    load_page(page_id(0), kc, vc);
  }
  for (int k = 0; k < my_count; ++k) {
    const int p = my_first + k * kDecWaves;
    if (k + 1 < my_count) {
      if (((k + 1) & 63) == 0) fetch_ids(k + 1);
      load_page(page_id(k + 1), kn, vn);
    }
    // Scores for 16 tokens x 16 head slots.
    f32x4 s = {};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = E::mma16(__builtin_bit_cast(typename E::vec8, kc[c]), qop[c], s);
    const int t0 = p * kPage;                 // first token of the page
    const int valid = min(kPage, len - t0);   // tokens of this page that exist
    if (valid < kPage) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * grp + i >= valid) s[i] = kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m2_new = m_new * a.c;
    const float m2_use = (m_new == kNegInf) ? 0.f : m2_new;
    const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m2_run - m2_new);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(fmaf(s[i], a.c, -m2_use));
    l_run = fmaf(alpha, l_run, (pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
    m2_run = m2_new;
    if (hs < G) {
      *reinterpret_cast<float4*>(&pbuf[wave][hs][4 * grp]) = make_float4(pr[0], pr[1], pr[2], pr[3]);
      if (grp == 0) abuf[wave][hs] = alpha;
    }
    // The writes above and the reads below are this wave's own LDS traffic;
    // LDS operations of one wave complete in order once issued.
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // acc[n][:] = alpha_n acc[n][:] + sum_t p[n][t] V[t][8e..8e+7]
    float vv[TPL][8];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const bool ok = r * TPL + i < valid;
      const uint32_t w[4] = {vc[i].x, vc[i].y, vc[i].z, vc[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv[i][2 * j] = ok ? E::to_f32(static_cast<uint16_t>(w[j] & 0xffffu)) : 0.f;
        vv[i][2 * j + 1] = ok ? E::to_f32(static_cast<uint16_t>(w[j] >> 16)) : 0.f;
      }
    }
#pragma unroll
    for (int n = 0; n < G; ++n) {
      const float al = abuf[wave][n];
      float pn[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) pn[i] = pbuf[wave][n][r * TPL + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = acc[n][j] * al;
#pragma unroll
        for (int i = 0; i < TPL; ++i) x = fmaf(pn[i], vv[i][j], x);
        acc[n][j] = x;
      }
    }
    if (k + 1 < my_count) {
#pragma unroll
      for (int c = 0; c < NC; ++c) kc[c] = kn[c];
#pragma unroll
      for (int i = 0; i < TPL; ++i) vc[i] = vn[i];
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // Wave totals: l over the four token groups, acc over the token rows.
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
#pragma unroll
  for (int n = 0; n < G; ++n)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = acc[n][j];
      if (RPI == 8) x += __uint_as_float(__builtin_amdgcn_update_dpp(
                         0u, __float_as_uint(x), 0x128, 0xf, 0xf, false));   // row_ror:8
      x = sum_xor16(x);
      x = sum_xor32(x);
      acc[n][j] = x;
    }
  if (lane < G) {
    wm[wave][lane] = m2_run;
    wl[wave][lane] = l_tot;
  }
  if (r == 0) {
#pragma unroll
    for (int n = 0; n < G; ++n)
#pragma unroll
      for (int j = 0; j < 8; ++j) wacc[wave][n][8 * e + j] = acc[n][j];
  }
  const bool bad = bad_len || __syncthreads_or(bad_page);

  // Merge the four wave states and write the chunk result.
  const bool final_out = nsplit == 1;
  for (int x = tid; x < G * D; x += kDecThreads) {
    const int n = x / D, dd = x % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w][n]);
    float lsum = 0.f, osum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float wt = exp2_fast(wm[w][n] - M);
        lsum = fmaf(wt, wl[w][n], lsum);
        osum = fmaf(wt, wacc[w][n][dd], osum);
      }
    }
    float o = lsum > 0.f ? osum / lsum : 0.f;
    float lse = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : kNegInf;
    if (bad) { o = nanf_(); lse = nanf_(); }
    const int h = hk * G + n;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    if (final_out) {
      store1(static_cast<OutT*>(a.o) + bh * D + dd, o);
      if (dd == 0) a.lse[bh] = lse;
    } else {
      a.part_o[(bh * a.max_splits + split) * D + dd] = o;
      if (dd == 0) a.part_lse[bh * a.max_splits + split] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per row.
// ---------------------------------------------------------------------------
struct MergeParams {
  const float* o_parts;
  const float* lse_parts;
  const int32_t* num_parts;   // per row, or NULL
  const int32_t* seq_lens;    // decode mode: parts per row from the split rule
  void* o;
  float* lse;
  int R, S, d;
  int heads;                  // decode mode: rows per sequence
  int fixed_splits;           // decode mode: num_splits argument
  int max_len;                // decode mode: max_pages * page_size
};

template <typename OutT, bool DECODE>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= a.R) return;
  int n;
  if (DECODE) {
    const int len = a.seq_lens[r / a.heads];
    const bool bad = len < 0 || len > a.max_len;
    n = decode_splits(bad ? 0 : len, a.fixed_splits);
    if (n <= 1) return;   // written directly by the decode kernel
  } else {
    n = a.num_parts ? a.num_parts[r] : a.S;
    n = max(0, min(n, a.S));
  }
  const float* lse_r = a.lse_parts + r * a.S;
  const float* o_r = a.o_parts + r * a.S * a.d;
  float M = kNegInf;
  bool has_nan = false;
  for (int c = 0; c < n; ++c) {
    const float v = lse_r[c];
    has_nan |= v != v;
    M = fmaxf(M, v);
  }
  OutT* out = static_cast<OutT*>(a.o) + r * a.d;
  if (has_nan) {   // a flagged part poisons the row instead of vanishing in the max
    for (int x = lane; x < a.d; x += 64) store1(out + x, nanf_());
    if (lane == 0) a.lse[r] = nanf_();
    return;
  }
  if (M == kNegInf) {
    for (int x = lane; x < a.d; x += 64) store1(out + x, 0.f);
    if (lane == 0) a.lse[r] = kNegInf;
    return;
  }
  float z = 0.f;
  for (int c = 0; c < n; ++c) z += expf(lse_r[c] - M);
  const float inv = 1.f / z;
  for (int x = lane; x < a.d; x += 64) {
    float s = 0.f;
    for (int c = 0; c < n; ++c) s = fmaf(expf(lse_r[c] - M), o_r[c * a.d + x], s);
    store1(out + x, s * inv);
  }
  if (lane == 0) a.lse[r] = M + logf(z);
}

template <typename OutT, bool DECODE>
hipError_t launch_merge_t(const MergeParams& p, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((p.R + 3) / 4);
  hipLaunchKernelGGL((merge_kernel<OutT, DECODE>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool DECODE>
hipError_t merge_dispatch(const MergeParams& p, fa_dtype out, hipStream_t s) {
  switch (out) {
    case FA_F32: return launch_merge_t<float, DECODE>(p, s);
    case FA_F16: return launch_merge_t<_Float16, DECODE>(p, s);
    case FA_BF16: return launch_merge_t<__bf16, DECODE>(p, s);
  }
  return hipErrorInvalidValue;
}

template <class E, typename OutT, int D>
hipError_t launch_decode_g(const DecParams& p, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<E, OutT, D, 1>), grid, dim3(kDecThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<E, OutT, D, 2>), grid, dim3(kDecThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<E, OutT, D, 4>), grid, dim3(kDecThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<E, OutT, D, 8>), grid, dim3(kDecThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E, typename OutT>
hipError_t launch_decode_d(const DecParams& p, int D, int G, dim3 grid, hipStream_t s) {
  return D == 64 ? launch_decode_g<E, OutT, 64>(p, G, grid, s)
                 : launch_decode_g<E, OutT, 128>(p, G, grid, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  DecParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_pool = static_cast<const uint16_t*>(a.k_pool);
  p.v_pool = static_cast<const uint16_t*>(a.v_pool);
  p.block_table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.o = a.o;
  p.lse = a.lse;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.B = a.B; p.H = a.H; p.Hkv = a.Hkv;
  p.max_pages = a.max_pages; p.num_pages = a.num_pages;
  p.num_splits = a.num_splits; p.max_splits = a.max_splits;
  p.c = a.scale * kLog2e;
  const int G = a.H / a.Hkv;
  const dim3 grid(a.max_splits, a.Hkv, a.B);
  hipError_t e;
  if (a.dtype == FA_BF16)
    e = a.out_dtype == FA_F32 ? launch_decode_d<BF16, float>(p, a.d, G, grid, s)
                              : launch_decode_d<BF16, __bf16>(p, a.d, G, grid, s);
  else
    e = a.out_dtype == FA_F32 ? launch_decode_d<F16, float>(p, a.d, G, grid, s)
                              : launch_decode_d<F16, _Float16>(p, a.d, G, grid, s);
  if (e != hipSuccess) return e;
  if (a.max_splits == 1) return hipSuccess;   // every sequence written directly
  MergeParams m;
  m.o_parts = a.part_o;
  m.lse_parts = a.part_lse;
  m.num_parts = nullptr;
  m.seq_lens = a.seq_lens;
  m.o = a.o;
  m.lse = a.lse;
  m.R = a.B * a.H;
  m.S = a.max_splits;
  m.d = a.d;
  m.heads = a.H;
  m.fixed_splits = a.num_splits;
  m.max_len = a.max_pages * kPage;
  return merge_dispatch<true>(m, a.out_dtype, s);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  MergeParams m;
  m.o_parts = a.o_parts;
  m.lse_parts = a.lse_parts;
  m.num_parts = a.num_parts;
  m.seq_lens = nullptr;
  m.o = a.o;
  m.lse = a.lse;
  m.R = a.R;
  m.S = a.S;
  m.d = a.d;
  m.heads = 1;
  m.fixed_splits = 0;
  m.max_len = 0;
  return merge_dispatch<false>(m, a.out_dtype, s);
}

}  // namespace fa
