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
// The decode is bound by HBM bandwidth, so the design is about keeping many
// bytes in flight per CU with little register cost:
//   * one workgroup (4 waves) per (sequence, KV head, chunk); wave w takes
//     pages w, w+4, ... of the chunk;
//   * each wave streams its pages through a private ring of kStages page
//     slots in LDS with direct-to-LDS loads (global_load_lds_dwordx4): the
//     next page is in flight while one is processed (two workgroups per CU,
//     so eight pages in flight per CU), and no VGPR holds data in transit.
//     The chunk's page ids are staged in LDS first;
//   * scores: S^T (16 tokens x 16 head slots) = K_page Q^T on one 16x16x32
//     matrix-core op per 32 of d; lane l holds head slot l % 16 for tokens
//     4(l/16) .. 4(l/16)+3, only the first G head slots are real;
//   * online softmax per head, two cross-row exchanges (l^16, l^32);
//   * P V on the matrix cores too, as O^T (16 d x 16 head slots) += V^T P^T
//     on 16x16x16 ops: the probabilities leave the score op in exactly the
//     layout of the P^T operand (lane l: head slot l % 16, tokens 4(l/16)
//     .. +3), so they never leave the registers; the V^T operand comes from
//     transposing LDS reads, and each head's rescale factor is in the lanes
//     that hold its accumulators;
//   * finally the 4 wave states are merged in LDS by the same rule and the
//     chunk's (o, lse) is written: as the output when the sequence has one
//     chunk, else as a partial for the merge kernel.
// Two score variants named in section "Paged and ragged layouts: FlashInfer"
// are runtime switches: a sliding window (only the newest `window` keys are
// visible; the chunks cover just those pages) and logit soft-capping (each
// scaled score x becomes cap * tanh(x / cap) before the softmax).
// Merge kernel, one wave per (sequence, head): M = max lse, weights e^(lse-M),
// fixed summation order, no atomics.
#include <mutex>

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_split_rule.hpp"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kPage = FA_PAGE_SIZE;   // 16 token slots per page
constexpr int kStages = 2;            // page slots per wave ring (2 workgroups fit a CU)
constexpr int kIdBatch = 1024;        // page ids staged in LDS at a time

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
  int group;             // H / Hkv: query heads sharing one KV head (<= head slots)
  float c;   // scale * log2(e)
  int window;            // > 0: only the newest `window` keys are visible
  int softcap_on;        // 1: scores are soft-capped
  float cap_over_scale;  // softcap / scale
  float scale_over_cap;  // scale / softcap
  // Ragged rows (the one-query sequences of a ragged forward batch): when
  // set, sequence b's query, O and LSE row is qo_indptr[b], and a sequence
  // with other than exactly one query row is left to the forward kernel.
  const int32_t* qo_indptr;
  int total_q;
};

// Keys visible to the query of a sequence of `len` cached tokens: positions
// [first_visible(len, window), len).
__device__ __forceinline__ int first_visible(int len, int window) {
  return (window > 0 && len > window) ? len - window : 0;
}


__device__ __forceinline__ float nanf_() { return __builtin_nanf(""); }

// K rows in the ring have their 16-byte chunks permuted by an XOR with
// kswz(row) so that the 16 lanes reading one chunk of 16 token rows hit 16
// different bank groups.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? row : (row >> 1) & 7;
}
// V rows likewise, so that the eight token rows one half-wave's transposing
// read touches (32 bytes of each) fall into different banks.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}

template <int D>
struct DecGeom {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per token row
  static constexpr int PAGE_ELEMS = kPage * D;       // one head's K (or V) of one page
  static constexpr int SLABS = PAGE_ELEMS * 2 / 1024; // 1 KiB wave-loads per tensor per page
  static constexpr int SLOT_ELEMS = 2 * PAGE_ELEMS;  // ring slot: K then V
  static constexpr int RING_ELEMS = kStages * SLOT_ELEMS;
  static constexpr int NC = D / 32;                  // 16x16x32 score steps over d
  static constexpr int NB = D / 16;                  // 16-wide d blocks of P V
};

// One wave's direct-to-LDS loads of one page (K then V of one KV head) into
// a ring slot.
template <int D>
struct PageLoader {
  using Geo = DecGeom<D>;
  int koff[Geo::SLABS], voff[Geo::SLABS];   // element offsets from the page base

  // Slab s of K fills ring slots 64s + lane (chunks permuted by kswz), of V
  // likewise (permuted by vswz).
  __device__ __forceinline__ PageLoader(int64_t row_stride, int lane) {
#pragma unroll
    for (int s = 0; s < Geo::SLABS; ++s) {
      const int slot = s * 64 + lane;
      const int row = slot / Geo::CPR, ch = slot % Geo::CPR;
      koff[s] = static_cast<int>(row * row_stride) + ((ch ^ kswz<D>(row)) * 8);
      voff[s] = static_cast<int>(row * row_stride) + ((ch ^ vswz<D>(row)) * 8);
    }
  }

  __device__ __forceinline__ void issue(const uint16_t* kbase, const uint16_t* vbase,
                                        int64_t page_stride, int page_id, uint16_t* slot) const {
    const int pg = __builtin_amdgcn_readfirstlane(page_id);
    const int64_t pbase = static_cast<int64_t>(pg) * page_stride;
    // Every cached byte is read exactly once: non-temporal loads keep the
    // stream from displacing anything useful in L2 / MALL.
    constexpr int kNonTemporal = 2;
#pragma unroll
    for (int s = 0; s < Geo::SLABS; ++s)
      load_lds16_policy<kNonTemporal>(kbase + pbase + koff[s], slot + s * 512);
#pragma unroll
    for (int s = 0; s < Geo::SLABS; ++s)
      load_lds16_policy<kNonTemporal>(vbase + pbase + voff[s], slot + Geo::PAGE_ELEMS + s * 512);
  }
};

// GP: head slots in use, a power of two >= the group size a.group (the
// remaining slots carry zero queries and are never stored).
template <class E, typename OutT, int D, int GP>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecParams a) {
  using Geo = DecGeom<D>;
  static_assert(GP >= 1 && GP <= 16, "head group must fit the 16 head slots");
  static_assert(kDecWaves * GP * D * 4 <= kDecWaves * Geo::RING_ELEMS * 2,
                "wave states must fit in the ring for the final merge");

  __shared__ __attribute__((aligned(16))) uint16_t ring[kDecWaves][Geo::RING_ELEMS];
  __shared__ int ids[kIdBatch];
  __shared__ float wm[kDecWaves][GP], wl[kDecWaves][GP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups u = S q + slot serve (sequence, KV head) pair q = b Hkv + hk,
  // the pairs in order; slot holds chunk (slot - q) mod S, so that the active
  // chunks 0 .. nsplit-1 of consecutive pairs start on consecutive XCDs (the
  // dispatcher sends workgroup u to XCD u % 8) and spread over all of them
  // whatever the sequences' chunk counts. Workgroups past a sequence's last
  // chunk leave at once.
  const int S = a.max_splits;
  const int u = static_cast<int>(blockIdx.x);
  const int pq = u / S, slot = u - pq * S;
  int split = slot - pq % S;
  if (split < 0) split += S;
  const int b = pq / a.Hkv, hk = pq - b * a.Hkv;
  const int G = a.group;
  int row = b;   // query / O / LSE row of the sequence
  if (a.qo_indptr) {
    const int qs = a.qo_indptr[b], qe = a.qo_indptr[b + 1];
    if (!(qs >= 0 && qe == qs + 1 && qe <= a.total_q)) return;   // whole workgroup: uniform
    row = qs;
  }
  const long long max_len = static_cast<long long>(a.max_pages) * kPage;
  const int len = a.seq_lens[b];
  const bool bad_len = len < 0 || len > max_len;
  const int kv_start = bad_len ? 0 : first_visible(len, a.window);
  const int nsplit = decode_splits(visible_tokens(len, a.window, max_len),
                                   decode_chunk_tokens(a.B, a.Hkv), a.max_splits, a.num_splits);
  if (split >= nsplit) return;                 // whole workgroup: uniform
  const int npages = bad_len ? 0 : (len + kPage - 1) / kPage;
  const int p0 = kv_start / kPage;             // first page holding a visible key
  int pb, pe;
  split_pages(npages - p0, nsplit, split, &pb, &pe);
  pb += p0;
  pe += p0;

  const int64_t row_stride = static_cast<int64_t>(a.Hkv) * D;   // between token slots
  const int64_t page_stride = row_stride * kPage;
  const uint16_t* kbase = a.k_pool + static_cast<int64_t>(hk) * D;
  const uint16_t* vbase = a.v_pool + static_cast<int64_t>(hk) * D;
  const int32_t* table = a.block_table + static_cast<int64_t>(b) * a.max_pages;

  // Q^T operand: lane l holds q[b, hk*G + l%16, 32c + 8(l/16) + j] (zero for
  // head slots >= G).
  const int hs = lane & 15, grp = lane >> 4;
  typename E::vec8 qop[Geo::NC];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(row) * a.H + hk * G + hs) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < Geo::NC; ++c) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (hs < G) u = *reinterpret_cast<const uint4*>(qrow + 32 * c);
      qop[c] = __builtin_bit_cast(typename E::vec8, u);
    }
  }

  const PageLoader<D> loader(row_stride, lane);
  // Per-lane read geometry. K operand of the scores: token hs, chunk
  // 4c + grp. V^T operand of P V block nb (d = 16 nb .. +15): the 16 lanes
  // of group grp read tokens 4 grp .. 4 grp + 3, lane hs supplying 4
  // elements of token 4 grp + hs / 4 at d = 16 nb + 4 (hs % 4); the
  // transposing read hands lane hs the 4 tokens of d = 16 nb + hs.
  uint16_t* my_ring = &ring[wave][0];
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(my_ring));
  const int vt = 4 * grp + (hs >> 2);
  uint32_t vaddr[Geo::NB];
#pragma unroll
  for (int nb = 0; nb < Geo::NB; ++nb)
    vaddr[nb] = ring_base + 2 * (Geo::PAGE_ELEMS + vt * D + 4 * (hs & 1) +
                                 (((2 * nb + ((hs & 3) >> 1)) ^ vswz<D>(vt)) * 8));

  // O^T accumulators: lane l holds head slot hs, d = 16 nb + 4 grp + i.
  f32x4 acc[Geo::NB];
#pragma unroll
  for (int nb = 0; nb < Geo::NB; ++nb) acc[nb] = f32x4{};
  float m_run = kNegInf, m2_run = kNegInf, l_run = 0.f;   // head slot hs
  bool bad_page = false;

  for (int b0 = pb; b0 < pe; b0 += kIdBatch) {
    const int bn = min(kIdBatch, pe - b0);
    if (b0 != pb) __syncthreads();   // previous batch's ids no longer read
    for (int x = tid; x < bn; x += kDecThreads) {
      int id = table[b0 + x];
      if (id < 0 || id >= a.num_pages) {   // outside the pool: never dereferenced
        bad_page = true;
        id = 0;
      }
      ids[x] = id;
    }
    __syncthreads();

    const int cnt = wave < bn ? (bn - wave + kDecWaves - 1) / kDecWaves : 0;
    for (int k = 0; k < min(kStages - 1, cnt); ++k)
      loader.issue(kbase, vbase, page_stride, ids[wave + k * kDecWaves],
                   my_ring + (k % kStages) * Geo::SLOT_ELEMS);

    for (int k = 0; k < cnt; ++k) {
      if (k + kStages - 1 < cnt) {
        const int kk = k + kStages - 1;
        loader.issue(kbase, vbase, page_stride, ids[wave + kk * kDecWaves],
                     my_ring + (kk % kStages) * Geo::SLOT_ELEMS);
      }
      // Wait for page k: the loads of the pages issued after it may stay
      // in flight (2 * SLABS instructions per page).
      const int after = min(kStages - 1, cnt - 1 - k);
      if (after >= 3) {
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * 2 * Geo::SLABS) : "memory");
      } else if (after == 2) {
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * 2 * Geo::SLABS) : "memory");
      } else if (after == 1) {
        __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * Geo::SLABS) : "memory");
      } else {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      const uint16_t* kl = my_ring + (k % kStages) * Geo::SLOT_ELEMS;
      const int p = b0 + wave + k * kDecWaves;   // page index within the sequence

      // Scores for 16 tokens x 16 head slots.
      f32x4 s = {};
#pragma unroll
      for (int c = 0; c < Geo::NC; ++c) {
        const auto op = *reinterpret_cast<const typename E::vec8*>(
            kl + hs * D + (((4 * c + grp) ^ kswz<D>(hs)) * 8));
        s = E::mma16(op, qop[c], s);
      }
      if (a.softcap_on) {
        // Soft-capped logit cap * tanh(scale * s / cap), kept in raw-score
        // units so that the base-2 step below stays one FMA.
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = a.cap_over_scale * tanhf(s[i] * a.scale_over_cap);
      }
      const int valid = min(kPage, len - p * kPage);   // tokens of this page that exist
      const int lo = kv_start - p * kPage;             // tokens before this are outside the window
      if (valid < kPage || lo > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * grp + i >= valid || 4 * grp + i < lo) s[i] = kNegInf;
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
      // P^T operand (zero for the padding head slots) and the rescale of
      // this lane's accumulators, whose head is its own.
      const i16x4 pop = hs < G ? E::pack4(pr[0], pr[1], pr[2], pr[3]) : i16x4{};
      if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
        for (int nb = 0; nb < Geo::NB; ++nb) acc[nb] *= alpha;
      }
      // V rows of tokens outside the visible range may hold anything (even
      // NaN): their operand elements are zeroed on the pages that have them.
      const uint32_t voff_slot = static_cast<uint32_t>((k % kStages) * Geo::SLOT_ELEMS * 2);
      if (valid < kPage || lo > 0) {
        int keep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) keep[j] = (4 * grp + j < valid && 4 * grp + j >= lo) ? -1 : 0;
#pragma unroll
        for (int nb = 0; nb < Geo::NB; ++nb) {
          i16x4 vop = lds_read_tr8(vaddr[nb] + voff_slot);
#pragma unroll
          for (int j = 0; j < 4; ++j) vop[j] &= static_cast<short>(keep[j]);
          acc[nb] = E::mma16k16(vop, pop, acc[nb]);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < Geo::NB; ++nb)
          acc[nb] = E::mma16k16(lds_read_tr8(vaddr[nb] + voff_slot), pop, acc[nb]);
      }
      // Every read of this slot is complete before the next iteration's
      // copies may refill it.
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }

  // Wave totals: l over the four token groups (acc already sums all tokens).
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
  // The ring is free once every wave has passed this barrier; the wave
  // states are merged in its memory.
  const bool bad = bad_len || __syncthreads_or(bad_page);
  float* wacc = reinterpret_cast<float*>(&ring[0][0]);   // [wave][G][D]
  if (lane < GP) {
    wm[wave][lane] = m2_run;
    wl[wave][lane] = l_tot;
  }
  if (hs < GP) {
#pragma unroll
    for (int nb = 0; nb < Geo::NB; ++nb)
      *reinterpret_cast<f32x4*>(&wacc[(wave * GP + hs) * D + 16 * nb + 4 * grp]) = acc[nb];
  }
  __syncthreads();

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
        osum = fmaf(wt, wacc[(w * GP + n) * D + dd], osum);
      }
    }
    float o = lsum > 0.f ? osum / lsum : 0.f;
    float lse = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : kNegInf;
    if (bad) { o = nanf_(); lse = nanf_(); }
    const int h = hk * G + n;
    const int64_t bh = static_cast<int64_t>(b) * a.H + h;
    if (final_out) {
      const int64_t rh = static_cast<int64_t>(row) * a.H + h;
      store1(static_cast<OutT*>(a.o) + rh * D + dd, o);
      if (dd == 0) a.lse[rh] = lse;
    } else {
      a.part_o[(bh * a.max_splits + split) * D + dd] = o;
      if (dd == 0) a.part_lse[bh * a.max_splits + split] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per row. The row's weights are formed once (lane c owns
// part c) and broadcast through LDS; every output element then sums its
// parts in index order.
// ---------------------------------------------------------------------------
struct MergeParams {
  const float* o_parts;
  const float* lse_parts;
  const int32_t* num_parts;   // per row, or NULL
  const int32_t* seq_lens;    // decode mode: parts per row from the split plan
  void* o;
  float* lse;
  int R, S, d;
  int heads;                  // decode mode: rows per sequence
  int Hkv;                    // decode mode: KV heads per sequence
  int B;                      // decode mode: sequences
  int fixed_splits;           // decode mode: num_splits argument
  long long max_len;          // decode mode: max_pages * page_size
  int window;                 // decode mode: visible-key window (0 = all)
  const float* o_extra;       // optional part S of every row: [R, d] ...
  const float* lse_extra;     // ... and [R] (NULL: none)
};

constexpr int kMergeMaxS = 1024;

// acc[i] += w_c o_c[x0 + i] for c = 0 .. n-1 in index order (i < V), the
// loads of 16 parts issued together.
template <int V>
__device__ __forceinline__ void merge_parts(const float* o_r, const float* w, int n, int d,
                                            int x0, float* acc) {
  for (int c0 = 0; c0 < n; c0 += 16) {
    float buf[16][V];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float* src = o_r + min(c0 + k, n - 1) * d + x0;
      if constexpr (V == 2) {
        const float2 t = *reinterpret_cast<const float2*>(src);
        buf[k][0] = t.x;
        buf[k][1] = t.y;
      } else {
        buf[k][0] = *src;
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool on = c0 + k < n;
      const float wk = w[min(c0 + k, n - 1)];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float t = fmaf(wk, buf[k][i], acc[i]);
        acc[i] = on ? t : acc[i];
      }
    }
  }
}

template <typename OutT, bool DECODE>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams a) {
  __shared__ float wsh[4][DECODE ? FA_MAX_SPLITS : kMergeMaxS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (r >= a.R) return;
  int n;
  if (DECODE) {
    n = decode_splits(visible_tokens(a.seq_lens[r / a.heads], a.window, a.max_len),
                      decode_chunk_tokens(a.B, a.Hkv), a.S, a.fixed_splits);
    if (n <= 1) return;   // written directly by the decode kernel
  } else {
    n = a.num_parts ? a.num_parts[r] : a.S;
    n = max(0, min(n, a.S));
  }
  const float* lse_r = a.lse_parts + r * a.S;
  const float* o_r = a.o_parts + r * a.S * a.d;
  OutT* out = static_cast<OutT*>(a.o) + r * a.d;

  // M = max over the parts; a NaN part poisons the row instead of vanishing
  // in the max.
  float M = kNegInf;
  bool has_nan = false;
  // The optional extra part: every lane reads it, so it enters the max and
  // the NaN check once per lane (both idempotent) and its weight is added
  // after the cross-lane sum.
  const float le = (!DECODE && a.lse_extra) ? a.lse_extra[r] : kNegInf;
  has_nan |= le != le;
  M = fmaxf(M, le);
  for (int c = lane; c < n; c += 64) {
    const float v = lse_r[c];
    has_nan |= v != v;
    M = fmaxf(M, v);
  }
  M = max_xor32(M);
#pragma unroll
  for (int sh = 16; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
  has_nan = __any(has_nan);
  if (has_nan || M == kNegInf) {
    const float fill = has_nan ? nanf_() : 0.f;
    for (int x = lane; x < a.d; x += 64) store1(out + x, fill);
    if (lane == 0) a.lse[r] = has_nan ? nanf_() : kNegInf;
    return;
  }
  float z = 0.f;
  for (int c = lane; c < n; c += 64) {
    const float w = expf(lse_r[c] - M);   // empty parts (-inf) weigh 0
    wsh[wave][c] = w;
    z += w;
  }
  z = sum_xor32(z);
#pragma unroll
  for (int sh = 16; sh >= 1; sh >>= 1) z += __shfl_xor(z, sh);
  const float we = le == kNegInf ? 0.f : expf(le - M);   // extra part's weight
  z += we;
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // own wave's LDS writes
  const float inv = 1.f / z;
  if (DECODE) {
    // d = 64 or 128: lane l sums elements l * d / 64 .. +d / 64 - 1 (one or
    // two) over the parts in index order. The part loads go out 16 at a time
    // (a short last batch re-reads the last part and skips its terms), so a
    // row of up to 64 parts waits for at most four round trips.
    float acc[2] = {0.f, 0.f};
    if (a.d == 128)
      merge_parts<2>(o_r, wsh[wave], n, 128, 2 * lane, acc);
    else
      merge_parts<1>(o_r, wsh[wave], n, 64, lane, acc);
    const int v = a.d >> 6;
    store1(out + v * lane, acc[0] * inv);
    if (v == 2) store1(out + v * lane + 1, acc[1] * inv);
  } else {
    for (int x = lane; x < a.d; x += 64) {
      float acc = 0.f;
      for (int c = 0; c < n; ++c) acc = fmaf(wsh[wave][c], o_r[c * a.d + x], acc);
      if (a.o_extra) acc = fmaf(we, a.o_extra[r * a.d + x], acc);
      store1(out + x, acc * inv);
    }
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
  if (G <= 1)
    hipLaunchKernelGGL((decode_kernel<E, OutT, D, 1>), grid, dim3(kDecThreads), 0, s, p);
  else if (G <= 2)
    hipLaunchKernelGGL((decode_kernel<E, OutT, D, 2>), grid, dim3(kDecThreads), 0, s, p);
  else if (G <= 4)
    hipLaunchKernelGGL((decode_kernel<E, OutT, D, 4>), grid, dim3(kDecThreads), 0, s, p);
  else if (G <= 8)
    hipLaunchKernelGGL((decode_kernel<E, OutT, D, 8>), grid, dim3(kDecThreads), 0, s, p);
  else if (G <= 16)
    hipLaunchKernelGGL((decode_kernel<E, OutT, D, 16>), grid, dim3(kDecThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class E, typename OutT>
hipError_t launch_decode_d(const DecParams& p, int D, int G, dim3 grid, hipStream_t s) {
  return D == 64 ? launch_decode_g<E, OutT, 64>(p, G, grid, s)
                 : launch_decode_g<E, OutT, 128>(p, G, grid, s);
}

constexpr int kMaxDevices = 64;

}  // namespace

// Partial results of fa_decode_paged_noalloc, for callers that cannot
// allocate: one buffer per device for the life of the process. Host code must
// never pass this name to a kernel or a copy (in host code it is a stand-in,
// not a device address); decode_scratch() hands out the device address.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

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
  p.group = a.H / a.Hkv;
  p.c = a.scale * kLog2e;
  p.window = a.window;
  p.softcap_on = a.softcap > 0.f ? 1 : 0;
  p.cap_over_scale = a.softcap > 0.f ? a.softcap / a.scale : 0.f;
  p.scale_over_cap = a.softcap > 0.f ? a.scale / a.softcap : 0.f;
  p.qo_indptr = nullptr;
  p.total_q = 0;
  const int G = a.H / a.Hkv;
  const dim3 grid(static_cast<unsigned>(a.max_splits * a.B * a.Hkv));
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
  m.Hkv = a.Hkv;
  m.B = a.B;
  m.fixed_splits = a.num_splits;
  m.max_len = static_cast<long long>(a.max_pages) * kPage;
  m.window = a.window;
  m.o_extra = nullptr;
  m.lse_extra = nullptr;
  return merge_dispatch<true>(m, a.out_dtype, s);
}

hipError_t launch_decode_rows(const ForwardPagedArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  DecParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_pool = static_cast<const uint16_t*>(a.k_pool);
  p.v_pool = static_cast<const uint16_t*>(a.v_pool);
  p.block_table = a.block_table;
  p.seq_lens = a.kv_lens;
  p.o = a.o;
  p.lse = a.lse;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  p.B = a.B; p.H = a.H; p.Hkv = a.Hkv;
  p.max_pages = a.max_pages; p.num_pages = a.num_pages;
  p.num_splits = 1; p.max_splits = 1;   // one workgroup per (sequence, KV head)
  p.group = a.H / a.Hkv;
  p.c = a.scale * kLog2e;
  p.window = 0;
  p.softcap_on = 0;
  p.cap_over_scale = 0.f;
  p.scale_over_cap = 0.f;
  p.qo_indptr = a.qo_indptr;
  p.total_q = a.total_q;
  const dim3 grid(static_cast<unsigned>(a.B * a.Hkv));
  if (a.dtype == FA_BF16)
    return a.out_dtype == FA_F32 ? launch_decode_d<BF16, float>(p, a.d, p.group, grid, s)
                                 : launch_decode_d<BF16, __bf16>(p, a.d, p.group, grid, s);
  return a.out_dtype == FA_F32 ? launch_decode_d<F16, float>(p, a.d, p.group, grid, s)
                               : launch_decode_d<F16, _Float16>(p, a.d, p.group, grid, s);
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
  m.Hkv = 1;
  m.B = 0;
  m.fixed_splits = 0;
  m.max_len = 0;
  m.window = 0;
  m.o_extra = a.o_extra;
  m.lse_extra = a.lse_extra;
  return merge_dispatch<false>(m, a.out_dtype, s);
}

}  // namespace fa
