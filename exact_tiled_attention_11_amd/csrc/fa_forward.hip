// Tiled attention forward for gfx950: online softmax over key tiles held in
// LDS, scores and the P V product on the matrix cores, causal tile skipping.
//
// The method is the one of "3.4 Attention Kernels", section "FlashAttention:
// tiling" (also "FlashAttention and Optimized Kernels", section "The online
// softmax"): each query row carries its largest score so far m, the sum l of
// its exponentials and the unnormalised output acc; per key tile compute the
// score tile, raise m,
// rescale l and acc by e^(m_old - m_new), add the tile's contribution; write
// O = acc / l and LSE = m + ln l once at the end (normalising once, as
// section "FlashAttention-2 and -3" describes). Key tiles wholly above the
// causal diagonal are never loaded.
//
// Work decomposition of the bf16/fp16 kernel (one workgroup = 8 waves, two
// per SIMD, 32 query rows per wave; 4 or 2 waves when the grid would not fill
// the chip; one key tile = 64 keys):
//   * Scores are computed transposed, S^T = K Q^T, so that every lane owns ONE
//     query row (l % 32) and 32 of the tile's keys: the row max and row sum
//     are in-lane reductions plus one exchange with lane l ^ 32, and the
//     per-row rescale factor is a lane-local scalar.
//   * The score accumulator, after exponentiation and rounding to the input
//     type, is directly the B operand of O^T += V^T P^T: no LDS round trip.
//     The contraction over keys uses the keys in the order the score layout
//     delivers them; V^T is fetched in that same key order.
//   * Each wave runs a software pipeline over the key tiles: one step turns
//     the scores of tile j into probabilities and adds P V(j), and in the
//     same instruction stream computes the scores of tile j+1 on the matrix
//     cores (see the comment at fwd16_kernel).
//   * K and V tiles are copied from global memory straight into LDS (no
//     register staging, from a wave-uniform base address plus per-lane
//     offsets), K two steps and V one step ahead. V stays row-major in LDS;
//     the transposed operand comes from ds_read_b64_tr_b16.
//   * Causal: a workgroup takes query blocks u and n-1-u of one head (the
//     second with its key tiles in descending order), so all workgroups stream
//     equally many tiles and those running together read the same tiles.
//   * Softmax runs in base 2 with scale*log2(e) folded into one FMA; m is
//     kept in raw-score units so LSE comes back in natural-log units.
// fp32 inputs use a 4-wave kernel on the 32x32x2 fp32 matrix-core op with P
// kept in fp32.
#include "fa_device.hpp"
#include "fa_internal.hpp"

#include <type_traits>

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQPW = 32;              // query rows per wave
constexpr int kBR = kWaves * kQPW;    // query rows per workgroup
constexpr int kBC = 64;               // keys per tile
// Largest growth (log2 units) of a row's max over the reference before the
// 16-bit kernel rescales: probabilities stay at or below 2^kLazy. bf16 and the
// fp32 sums hold 2^32 with room to spare; fp16 (largest finite 65504) needs a
// bound under 2^16.
template <class E>
constexpr float kLazy = std::is_same<E, BF16>::value ? 32.f : 8.f;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Nq, Nk;
  int group;       // H / Hkv
  int n_qblocks;   // query blocks per (batch, head)
  int units;       // workgroup work units per (batch, head)
  int total;       // workgroups in the grid
  float c;         // scale * log2(e)
  int off;         // Nk - Nq: key j is visible to query i iff j <= i + off
  // Ragged queries over a paged cache (K/V point at the page pools):
  const int32_t* qo_indptr;    // [B + 1]: rows of sequence b are qo_indptr[b] ..
                               //   (NULL: one sequence owning all total_q rows)
  const int32_t* kv_lens;      // [B] (NULL: every sequence has fixed_kv_len keys)
  const int32_t* block_table;  // [B, max_pages]
  int max_pages, num_pages, total_q, max_q_len, fixed_kv_len;
  // Partial mode (non-causal, part_o != NULL): each query block is processed
  // by kv_splits workgroups over near-equal key-tile ranges, each writing an
  // fp32 partial (o, lse) to part_o [total_q * H, kv_splits, D] and
  // part_lse [total_q * H, kv_splits] instead of O and LSE.
  int kv_splits;
  float* part_o;
  float* part_lse;
  // 1: sequences with exactly one query row are left to the decode kernel.
  int skip_single;
};

// ---------------------------------------------------------------------------
// bf16 / fp16 inputs: 32x32x16 matrix-core ops, K/V tiles loaded straight
// into LDS (no register staging), 2 waves per SIMD.
// ---------------------------------------------------------------------------

// LDS tiles are unpadded [kBC rows][D] with the 16-byte chunks of each row
// permuted by an XOR with swz(row), so that both the K operand reads (16
// lanes x 16 B per cycle, 16 consecutive rows) and the transposed V reads
// (32 lanes x 8 B per cycle, 4 rows x 4 chunks) hit 64 distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return 4 * (row & 3) + ((row >> 2) & 3);
  } else {
    const int b = (row >> 1) & 7;
    return ((b & 1) << 2) | (b & 2) | ((b >> 2) & 1);
  }
}

// This wave's share of one K or V tile load, straight into LDS. Slab s covers
// the LDS chunk slots 64s .. 64s+63 (1 KiB); lane l fills slot 64s + l with
// the global 16-byte chunk (slot % CPR) ^ swz(row) of key row slot / CPR.
template <int D, int NW>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int SPW = kBC * CPR / 64 / NW;   // slabs per wave per tensor
  uint32_t voff[SPW];   // byte offset of this lane's chunk from key row k0
  int row[SPW];
  int chunk[SPW];       // element offset of the chunk within its key row
  uint32_t lds0;        // byte offset of this wave's first slab in a tile (wave-uniform)

  __device__ __forceinline__ TileLoader(int64_t rs, int wave, int lane) {
    const int slab0 = wave * SPW;
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
      const int slot = (slab0 + r) * 64 + lane;
      row[r] = slot / CPR;
      chunk[r] = ((slot % CPR) ^ swz<D>(row[r])) * 8;
      voff[r] = static_cast<uint32_t>((row[r] * rs + chunk[r]) * 2);
    }
    lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(slab0 * 1024));
  }

  // Copies of this wave's slabs of the tile at key k0 into the tile at LDS
  // byte address `lds`, from the wave-uniform row k0 plus per-lane offsets.
  // Rows past the last key re-read the last key (finite data whose scores
  // are masked to -inf, i.e. weight 0); only the ragged last tile needs it.
  __device__ __forceinline__ void load(const uint16_t* base, int64_t rs, int k0, int nk,
                                       uint32_t lds) const {
    const uint16_t* b0 = base + static_cast<int64_t>(k0) * rs;
    if (__builtin_expect(k0 + kBC > nk, 0)) {
      load_clamped(b0, rs, nk - k0, lds);
    } else {
#pragma unroll
      for (int r = 0; r < SPW; ++r) load_lds16_sbase(b0, voff[r], lds + lds0 + r * 1024);
    }
  }
  // The copies of a tile with only `left` (< kBC) keys from its first row b0
  // to the end of the sequence.
  __device__ __forceinline__ void load_clamped(const uint16_t* b0, int64_t rs, int left,
                                               uint32_t lds) const {
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
      uint32_t vo = static_cast<uint32_t>((min(row[r], left - 1) * rs + chunk[r]) * 2);
      __asm__("" : "+v"(vo));   // computed only on this (rare) path
      load_lds16_sbase(b0, vo, lds + lds0 + r * 1024);
    }
  }

  // Bytes a buffer resource whose base is a tile's first row must cover for
  // `rows` (1..kBC) rows of keys: rows past the range are out of range and
  // copy as zeros without a memory access. (rows - 1) * rs + D <= Nk * rs
  // elements, below 2^31 (the API's size limit), so the count fits 32 bits.
  static __device__ __forceinline__ uint32_t rsrc_bytes(int rs, int rows) {
    return static_cast<uint32_t>((rows - 1) * rs + D) * 2u;
  }
  // Slab r of this wave's share of the tile of resource t.
  __device__ __forceinline__ void load_buf(i32x4 t, int r, uint32_t lds) const {
    load_lds16_buf(t, voff[r], lds + lds0 + r * 1024);
  }
};

// The same share of a K or V tile when the keys live in 16-token pages: key
// k0 + row is slot row % 16 of the tile's page row / 16 (a 64-key tile spans
// four pages). A wave's slabs cover kBC / NW consecutive rows, all inside one
// page (page WAVE_ROWS * wave / 16 of the tile), so one page id per wave and
// tile addresses them.
constexpr int kPageTokens = FA_PAGE_SIZE;

template <int D, int NW>
struct PagedTileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int RPS = 64 / CPR;                 // key rows per slab
  static constexpr int SPW = kBC * CPR / 64 / NW;
  static constexpr int WAVE_ROWS = SPW * RPS;
  static_assert(WAVE_ROWS * NW == kBC && kPageTokens % WAVE_ROWS == 0,
                "a wave's slabs must lie in one page");
  uint32_t voff[SPW];   // byte offset of this lane's chunk from the start of its page
  uint32_t lds0;        // byte offset of this wave's first slab in a tile (wave-uniform)

  __device__ __forceinline__ PagedTileLoader(int64_t rs, int wave, int lane) {
    const int slab0 = wave * SPW;
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
      const int slot = (slab0 + r) * 64 + lane;
      const int row = slot / CPR;
      const int coff = ((slot % CPR) ^ swz<D>(row)) * 8;
      voff[r] = static_cast<uint32_t>(((row % kPageTokens) * rs + coff) * 2);
    }
    lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(slab0 * 1024));
  }
  // Which of a tile's four pages holds this wave's rows.
  static __device__ __forceinline__ int page_of_wave(int wave) {
    return wave * WAVE_ROWS / kPageTokens;
  }
};

// Work unit of the 16-bit kernel. Non-causal: one query block. Causal: the
// query blocks u and n-1-u of one (batch, head), one after the other, the
// short one with keys in ascending tile order and the long one in descending
// order. Every unit then streams the same number of key tiles, and at step g
// all units of a head read either tile g or the one same tile counted from the
// other end, so the concurrently running units of a head share their K/V
// tiles in L2. The order of the key tiles does not change the result of the
// online softmax (up to rounding).
__device__ __forceinline__ int tile_count(int last_key) { return last_key >= 0 ? last_key / kBC + 1 : 0; }

template <int P>
using Parity = std::integral_constant<int, P>;

// Software pipeline of one wave over the key tiles of a query block. Step j
// turns the scores of tile j (computed at step j-1) into probabilities and
// adds P V(j) to the output accumulator, and in the same instruction stream
// computes the scores of tile j+1 on the matrix cores: the exponentials of
// one tile run between the score products of the next, and the packing and
// row sums between the P V products, in the same wave. (On CDNA4 vector work
// hides behind matrix-core work of its own wave; spread over two waves of
// one SIMD the two kinds of work mostly serialise.)
//
// LDS: K tiles in a 2-slot ring filled two steps ahead, V tiles in a 2-slot
// ring filled one step ahead; counting the steps of a segment (one query
// block) from 0, K of step x lives in K slot x & 1 and V of step x in V slot
// x & 1. Step j reads K slot (j+1) & 1 and V slot j & 1 and issues the copies
// of K(j+2) into K slot j & 1 and of V(j+1) into V slot (j+1) & 1, both freed
// by the barrier that ends step j-1 (dense layout: between its first score
// products; paged: at its top). The rings restart with every segment.
// Every step is compiled once per parity of j, so that all LDS addresses are
// per-lane constants plus immediate offsets. With 16-bit outputs a further
// per-wave LDS tile carries O on its way out, so that it is stored as whole
// rows.
template <class E, typename OutT, int D, bool CAUSAL, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64, (NW == 4 && D == 128) ? 1 : NW == 2 ? 2 : 8 / NW)
void fwd16_kernel(const FwdParams a) {
  constexpr int TILE = kBC * D;                 // elements per K or V tile
  constexpr int QF = D / 16;
  constexpr int DB = D / 32;
  constexpr int BR = NW * kQPW;
  using V8 = typename E::vec8;
  // the paged share of a tile (instantiated for the dense layout too, unused)
  using PLoader = PagedTileLoader<D, PAGED ? NW : 8>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[4][TILE];   // K0 K1 V0 V1
  // 16-bit outputs: each wave's 32 x D tile of O passes through LDS so that
  // it is stored as whole rows.
  constexpr bool kStageO = sizeof(OutT) == 2;
  __shared__ __attribute__((aligned(16))) uint16_t ostage[kStageO ? NW * kQPW * D : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bh, u;
  xcd_group_unit(static_cast<int>(blockIdx.x), a.B * a.Hkv, a.units, &bh, &u);
  if (bh < 0) return;   // padding of the grid: whole workgroup
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int G = a.group;   // query heads per KV head

  // Sequence geometry: Nq query rows starting at row q_row0 of Q and O, Nk keys.
  // The workgroup serves KV head hk; its rows are the packed pairs (query i,
  // head hk*G + g), row r = i*G + g, so every K/V tile is loaded once for the
  // whole head group and a short query (a decode token) fills G rows, not a
  // block.
  int Nq, Nk, nqb;
  int64_t q_row0;
  bool bad = false;   // device-side contract violation: this sequence's outputs are NaN
  if constexpr (PAGED) {
    const int qs = a.qo_indptr ? a.qo_indptr[b] : 0;
    const int qe = a.qo_indptr ? a.qo_indptr[b + 1] : a.total_q;
    if (qs < 0 || qe < qs || qe > a.total_q) return;   // rows unknown: nothing is written
    if (a.skip_single && qe == qs + 1) return;           // a decode row: the decode kernel's
    Nq = qe - qs;
    q_row0 = qs;
    Nk = a.kv_lens ? a.kv_lens[b] : a.fixed_kv_len;
    if (Nk < 0 || Nk > a.max_pages * kPageTokens || Nq > a.max_q_len) {
      bad = true;
      Nk = 0;
    }
  } else {
    Nq = a.Nq;
    Nk = a.Nk;
    q_row0 = static_cast<int64_t>(b) * a.Nq;
  }
  const int nrows = Nq * G;   // packed rows of this (sequence, KV head)
  nqb = (nrows + BR - 1) / BR;
  const int off = Nk - Nq;
  // Partial mode (paged, non-causal, part_o set): unit = query unit *
  // kv_splits + split, and each split writes an fp32 partial (o, lse).
  const bool partial = PAGED && !CAUSAL && a.part_o != nullptr;
  const int S = partial ? a.kv_splits : 1;
  const int uq = S > 1 ? u / S : u;
  const int split = u - uq * S;
  if (uq >= (CAUSAL ? (nqb + 1) / 2 : nqb)) return;   // whole workgroup: uniform

  const int qb_first = uq;
  const int qb_second = CAUSAL ? nqb - 1 - uq : uq;
  const int nseg = (CAUSAL && qb_second > qb_first) ? 2 : 1;
  auto block_tiles = [&](int qb) {
    int last = Nk - 1;
    // the query of the block's last packed row (a block may end inside a
    // query's group of heads when G does not divide BR)
    if (CAUSAL) last = min(last, (min(qb * BR + BR, nrows) - 1) / G + off);
    return tile_count(last);
  };
  int n0 = block_tiles(qb_first);
  int t_begin = 0;   // first key tile of this split
  if (S > 1) {       // near-equal tile ranges, the first n0 % S one tile longer
    const int q = n0 / S, r = n0 % S;
    t_begin = split * q + min(split, r);
    n0 = q + (split < r ? 1 : 0);
  }
  const int n1 = nseg == 2 ? block_tiles(qb_second) : 0;
  const int n_steps = n0 + n1;
  // Key tile streamed at step g: ascending through the first block, then
  // descending through the second.
  auto tile_at = [&](int g) { return g < n0 ? t_begin + g : n_steps - 1 - g; };

  const int64_t q_rs = static_cast<int64_t>(a.H) * D;
  const int64_t kv_rs = static_cast<int64_t>(a.Hkv) * D;
  const int kv_rs32 = a.Hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + static_cast<int64_t>(hk) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + static_cast<int64_t>(hk) * D;
  if constexpr (!PAGED) {
    kbase += static_cast<int64_t>(b) * a.Nk * kv_rs;
    vbase += static_cast<int64_t>(b) * a.Nk * kv_rs;
  }
  // Paged: a wave's share of a 64-key tile lies in one 16-token page (page
  // wave / 2 of the tile's four), so each copy needs one page id per wave,
  // read from the block table by a scalar load one step before the copy is
  // issued. A page past the sequence's last one is never read (its resource
  // covers no rows); an id outside the pool is replaced by page 0 and marks
  // the sequence bad (NaN output, agreed over all waves at the end). The
  // page index (wave-uniform) and the page's byte offset (below 2^32: the API
  // limits a pool to 2^31 elements) keep this bookkeeping in scalar registers.
  const int32_t* table = PAGED ? a.block_table + static_cast<int64_t>(b) * a.max_pages : nullptr;
  const int last_page = Nk > 0 ? (Nk - 1) / kPageTokens : 0;
  const int wave_page = __builtin_amdgcn_readfirstlane(PLoader::page_of_wave(wave));
  const uint32_t page_bytes = static_cast<uint32_t>(kv_rs32 * kPageTokens * 2);
  bool bad_page = false;
  // The id as loaded (a vector register, the same in every lane); made
  // wave-uniform only where it is used, a step later, so that the load's
  // latency hides behind that step instead of stalling this one.
  auto fetch_id = [&](int t) { return table[min(t * 4 + wave_page, last_page)]; };
  auto load_id = [&](int t) { return __builtin_amdgcn_readfirstlane(fetch_id(t)); };
  // Buffer resource over the rows of this wave's page of key tile t that
  // hold keys (none past the sequence's last key: those copy as zeros).
  auto page_rsrc = [&](const uint16_t* base, int id, int t) {
    const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(a.num_pages);
    bad_page = bad_page || !ok;
    const uint32_t pid = ok ? static_cast<uint32_t>(id) : 0u;
    const int valid = min(max(Nk - (t * kBC + wave_page * kPageTokens), 0), kPageTokens);
    return buffer_rsrc(reinterpret_cast<const uint8_t*>(base) + pid * page_bytes,
                       valid > 0 ? static_cast<uint32_t>((valid - 1) * kv_rs32 + D) * 2u : 0u);
  };

  // Per-lane LDS read addresses (bytes, LDS address space) in the first K
  // slot; other slots and key rows are immediate offsets from these.
  // K operand of score step c, keys 0..31: row kr, chunk (2c + khi) ^ swz(kr);
  // keys 32..63 are 32 rows further.
  const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&smem[0][0]));
  const int kr = lane & 31;
  const int khi = lane >> 5;
  uint32_t kaddr[QF];
#pragma unroll
  for (int c = 0; c < QF; ++c)
    kaddr[c] = sbase + 2 * (kr * D + (((2 * c + khi) ^ swz<D>(kr)) * 8));
  // Opaque to the optimiser, so every read uses the full per-lane address
  // plus an immediate offset instead of re-adding a common base per step.
#pragma unroll
  for (int c = 0; c < QF; ++c) __asm__("" : "+v"(kaddr[c]));
  // V^T operand of d block db (transposed 4x4 reads): rows vrow and vrow + 8
  // of each 16-key group.
  const int blk = lane >> 4, r16 = lane & 15;
  const int vrow = 4 * (blk >> 1) + (r16 >> 2);          // 0..7
  const int vcl = 2 * (blk & 1) + ((r16 & 3) >> 1);      // chunk within a 32-wide d block
  const int vin = (r16 & 1) * 4;                          // element within the chunk
  uint32_t vaddr0[DB], vaddr1[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    vaddr0[db] = sbase + 2 * (vrow * D + vin + (((4 * db + vcl) ^ swz<D>(vrow)) * 8));
    vaddr1[db] = sbase + 2 * ((vrow + 8) * D + vin + (((4 * db + vcl) ^ swz<D>(vrow + 8)) * 8));
    __asm__("" : "+v"(vaddr0[db]), "+v"(vaddr1[db]));
  }
  constexpr uint32_t kSlotBytes = TILE * 2;   // slot x of smem starts x * kSlotBytes in

  const TileLoader<D, NW> loader(kv_rs, wave, lane);
  const PLoader ploader(kv_rs, wave, lane);
  // Paged: page id of the tile whose V is copied next (= the K tile of the
  // previous step) and, as fetched, of the K tile copied next.
  int id_v = 0, raw_k = 0;
  auto copy_k = [&](int g, uint32_t dst) { loader.load(kbase, kv_rs, tile_at(g) * kBC, Nk, dst); };
  auto copy_v = [&](int g, uint32_t dst) { loader.load(vbase, kv_rs, tile_at(g) * kBC, Nk, dst); };
  // This wave's slabs of a paged tile, from a page resource.
  auto copy_paged = [&](i32x4 rsrc, uint32_t dst) {
#pragma unroll
    for (int r = 0; r < PLoader::SPW; ++r)
      load_lds16_buf(rsrc, ploader.voff[r], dst + ploader.lds0 + r * 1024);
  };
  // First copies of a segment whose first step is g: K and V of step g into
  // slot 0, K of step g + 1 into K slot 1 (when the segment has it).
  auto segment_copies = [&](int g, int nt) {
    if (nt <= 0) return;
    if constexpr (PAGED) {
      const int t0 = tile_at(g);
      const int id0 = load_id(t0);
      copy_paged(page_rsrc(kbase, id0, t0), sbase);
      copy_paged(page_rsrc(vbase, id0, t0), sbase + 2 * kSlotBytes);
      if (nt > 1) {
        id_v = load_id(tile_at(g + 1));
        copy_paged(page_rsrc(kbase, id_v, tile_at(g + 1)), sbase + kSlotBytes);
        if (nt > 2) raw_k = fetch_id(tile_at(g + 2));
      }
    } else {
      copy_k(g, sbase);
      copy_v(g, sbase + 2 * kSlotBytes);
      if (nt > 1) copy_k(g + 1, sbase + kSlotBytes);
    }
  };

  // Scores of two key tiles; sc0 holds the tiles of the even steps of a
  // segment, sc1 those of its odd steps.
  f32x16 sc0[2], sc1[2];
  f32x16 acc[DB];
  // This lane's query row: reference max m_run (raw score units) and m2_run =
  // m_run * scale * log2(e); l_run = sum of 2^(s c - m2_run) over the keys
  // so far; lt_run = the same sum over the values rounded to the input type,
  // as the P V products use them.
  float m_run, m2_run, l_run, lt_run;
  typename E::vec8 qf[QF];      // Q^T operand: lane l holds Q[row][16c + 8(l/32) .. +8]

  // Scores S^T = K Q^T of the K tile in slot ks (no interleaving).
  auto scores = [&](uint32_t ks, f32x16* s) {
    const uint32_t o0 = ks * kSlotBytes, o1 = o0 + 32 * D * 2;
    s[0] = f32x16{};
    s[1] = f32x16{};
    V8 a0 = lds_read16<V8>(kaddr[0] + o0);
    V8 a1 = lds_read16<V8>(kaddr[0] + o1);
#pragma unroll
    for (int c = 0; c < QF; ++c) {
      V8 n0v = a0, n1v = a1;
      if (c + 1 < QF) {
        n0v = lds_read16<V8>(kaddr[c + 1] + o0);
        n1v = lds_read16<V8>(kaddr[c + 1] + o1);
      }
      s[0] = E::mma32(a0, qf[c], s[0]);
      s[1] = E::mma32(a1, qf[c], s[1]);
      a0 = n0v;
      a1 = n1v;
    }
  };

  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
  };

  // Copies of one step in the contiguous layout: this wave's slabs of the K
  // tile of resource kt into the K slot at LDS byte address kl, and of the V
  // tile vt into vl.
  struct StepCopies {
    i32x4 kt, vt;
    uint32_t kl, vl;
  };
  // Issue copy x of the step's 2 * SPW copies (K slabs first).
  auto issue_copy = [&](const StepCopies& cp, int x) {
    constexpr int SPW = TileLoader<D, NW>::SPW;
    if constexpr (PAGED) {
      if (x < SPW)
        load_lds16_buf(cp.kt, ploader.voff[x], cp.kl + ploader.lds0 + x * 1024);
      else
        load_lds16_buf(cp.vt, ploader.voff[x - SPW], cp.vl + ploader.lds0 + (x - SPW) * 1024);
    } else {
      if (x < SPW)
        loader.load_buf(cp.kt, x, cp.kl);
      else
        loader.load_buf(cp.vt, x - SPW, cp.vl);
    }
  };

  // One pipelined step: scores of the next tile into `nx` (K slot ks),
  // probabilities of `cur`, P V with the V tile in slot vs. The source order
  // is the instruction order wanted: each score product is followed by two
  // exponentials (with their argument FMAs) and the next K operand read, each
  // P V product by the packing and row-sum work of its neighbours and the V
  // operand reads of the next product. With CP, the step's K/V copies `cp`
  // are issued one by one between the first score products: issued together
  // at the top of the step, the copies of all waves queue behind each other
  // in the memory pipeline and every wave waits for its turn.
  auto fused = [&](uint32_t ks, uint32_t vs, f32x16* cur, f32x16* nx, float m2, auto with_copies,
                   const StepCopies& cp) {
    constexpr bool CP = decltype(with_copies)::value;
    constexpr int NCP = 2 * TileLoader<D, NW>::SPW;   // copies per step
    constexpr int EPS = 32 / (2 * QF);   // exponentials per score product
    const uint32_t o0 = ks * kSlotBytes, o1 = o0 + 32 * D * 2;
    nx[0] = f32x16{};
    nx[1] = f32x16{};
    V8 a0 = lds_read16<V8>(kaddr[0] + o0);
    V8 a1 = lds_read16<V8>(kaddr[0] + o1);
#pragma unroll
    for (int c = 0; c < QF; ++c) {
      V8 n0v = a0, n1v = a1;
      if (c + 1 < QF) n0v = lds_read16<V8>(kaddr[c + 1] + o0);
      nx[0] = E::mma32(a0, qf[c], nx[0]);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int x = 2 * c * EPS + e;   // 0..31
        cur[x >> 4][x & 15] = exp2_fast(fmaf(cur[x >> 4][x & 15], a.c, -m2));
      }
      if (c + 1 < QF) n1v = lds_read16<V8>(kaddr[c + 1] + o1);
      nx[1] = E::mma32(a1, qf[c], nx[1]);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int x = (2 * c + 1) * EPS + e;
        cur[x >> 4][x & 15] = exp2_fast(fmaf(cur[x >> 4][x & 15], a.c, -m2));
      }
      if constexpr (CP) {
#pragma unroll
        for (int x = 0; x < NCP; ++x)
          if (c == x * (QF / 2) / NCP) issue_copy(cp, x);
      }
      a0 = n0v;
      a1 = n1v;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int c = 0; c < 2 * QF; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 2 * EPS, 0);
      if (c + 2 < 2 * QF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // P V: product (kb, hh, db) uses pb[2kb + hh]; the operands of a pair
    // (kb, hh) are packed just before its first product. Two row sums
    // accumulate between the products: of the probabilities (for the LSE)
    // and of the rounded operands the products use (for normalising O).
    float r0 = 0.f, r1 = 0.f, t0 = 0.f;
    V8 pb;
    i16x4 lo = lds_read_tr8(vaddr0[0] + vs * kSlotBytes);
    i16x4 hi = lds_read_tr8(vaddr1[0] + vs * kSlotBytes);
#pragma unroll
    for (int m = 0; m < 4 * DB; ++m) {
      const int kb = m / (2 * DB), hh = (m / DB) & 1, db = m % DB;
      if (db == 0) {
        const int o = 8 * hh;
        pb = pack8<E>(cur[kb][o + 0], cur[kb][o + 1], cur[kb][o + 2], cur[kb][o + 3],
                      cur[kb][o + 4], cur[kb][o + 5], cur[kb][o + 6], cur[kb][o + 7]);
      }
      i16x4 nlo = lo, nhi = hi;
      if (m + 1 < 4 * DB) {
        const int kb1 = (m + 1) / (2 * DB), hh1 = ((m + 1) / DB) & 1, db1 = (m + 1) % DB;
        const uint32_t o = vs * kSlotBytes + (32 * kb1 + 16 * hh1) * D * 2;
        nlo = lds_read_tr8(vaddr0[db1] + o);
        nhi = lds_read_tr8(vaddr1[db1] + o);
      }
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[db] = E::mma32(__builtin_bit_cast(V8, w), pb, acc[db]);
      // Row sums: the 32 probabilities spread over the 4 DB products, the 8
      // rounded operands of pb over its DB products.
#pragma unroll
      for (int e = 0; e < 32 / (4 * DB); ++e) {
        const int x = m * (32 / (4 * DB)) + e;
        if (e & 1) r1 += cur[x >> 4][x & 15]; else r0 += cur[x >> 4][x & 15];
      }
#pragma unroll
      for (int e = db * 4 / DB; e < (db + 1) * 4 / DB; ++e) t0 = E::sum2(pb, e, t0);
      lo = nlo;
      hi = nhi;
    }
    return make_float2(r0 + r1, t0);
  };

  int g = 0;   // step counter over both blocks
  for (int seg = 0; seg < nseg; ++seg) {
    const int qb = seg == 0 ? qb_first : qb_second;
    const int nt = seg == 0 ? n0 : n1;
    const int qw0 = qb * BR + wave * kQPW;   // first packed row of this wave
    const int prow = qw0 + (lane & 31);      // this lane's packed row
    const int qrow = prow / G;               // its query position ...
    const int h = hk * G + (prow - qrow * G);   // ... and query head
    // Last key any row of this wave sees; -1 for a wave without real rows.
    const int wave_last = qw0 >= nrows ? -1
                          : CAUSAL ? min(Nk - 1, (min(qw0 + kQPW, nrows) - 1) / G + off)
                                   : Nk - 1;
    const int lim_row = CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1;   // this lane's last key
    // A tile starting at key k0 holds keys some row of this wave must not see
    // (past the last key, or past the diagonal of the wave's first row) iff
    // k0 > mask_k0.
    const int mask_k0 = __builtin_amdgcn_readfirstlane(
        CAUSAL ? min(Nk - kBC, qw0 / G + off - kBC + 1) : Nk - kBC);

    // The LDS rings restart with every segment (its step j uses the slots of
    // parity j & 1): first copies, then this segment's query fragments.
    segment_copies(g, nt);
    // Key tile of the current step: up by one per step through the first
    // block and down through the second.
    const int dt = seg == 0 ? 1 : -1;
    int tcur = nt > 0 ? tile_at(g) : 0;
    // Contiguous layout: at step j, the V tile copied (that of step j + 1)
    // starts toff bytes after vbase and the K tile (of step j + 2) toff bytes
    // after kb2, one tile stride past kbase; toff moves by one stride per
    // step (below 2^32: the API limits a tensor to 2^31 elements; past a
    // segment's ends it wraps, but those copies cover no bytes). Every tile
    // of a segment is whole but the one holding the last key when Nk is not
    // a multiple of the tile, streamed at step j_rag of the segment (if at
    // all): its resource covers only the rows up to the last key.
    const int64_t dstep = static_cast<int64_t>(dt) * kBC * kv_rs;
    const uint8_t* kb2 = reinterpret_cast<const uint8_t*>(kbase) + dstep * 2;
    const uint8_t* vb1 = reinterpret_cast<const uint8_t*>(vbase);
    uint32_t toff = static_cast<uint32_t>(static_cast<int64_t>(tcur + dt) * kBC * kv_rs * 2);
    const uint32_t dstep_b = static_cast<uint32_t>(dstep * 2);
    const uint32_t full_bytes = TileLoader<D, NW>::rsrc_bytes(kv_rs32, kBC);
    const int t_rag = (Nk % kBC) ? Nk / kBC : -1;
    int j_rag = t_rag < 0 ? -1 : dt > 0 ? t_rag - tcur : tcur - t_rag;
    if (j_rag >= nt) j_rag = -1;
    const uint32_t rag_bytes =
        t_rag < 0 ? full_bytes : TileLoader<D, NW>::rsrc_bytes(kv_rs32, Nk - t_rag * kBC);
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           (q_row0 + qrow) * q_rs +
                           static_cast<int64_t>(h) * D + 8 * (lane >> 5);
#pragma unroll
      for (int c = 0; c < QF; ++c) {
        uint4 v4 = make_uint4(0, 0, 0, 0);
        if (qrow < Nq) v4 = *reinterpret_cast<const uint4*>(qp + 16 * c);
        qf[c] = __builtin_bit_cast(typename E::vec8, v4);
      }
    }
    // Consuming the fragments here makes the compiler wait for their loads
    // once, instead of at every score product of the loop.
#pragma unroll
    for (int c = 0; c < QF; ++c) __asm__ volatile("" : "+v"(qf[c]));
    __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    m_run = kNegInf;
    m2_run = kNegInf;
    l_run = 0.f;
    lt_run = 0.f;

    // Scores of the segment's first tile, then a barrier: the first step
    // refills the K slot they were read from.
    bool cur_ok = nt > 0 && tile_at(g) * kBC <= wave_last;
    if (cur_ok) scores(0, sc0);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Step j of the segment (global step g).
    auto step = [&](auto par, int j) {
      constexpr int P = decltype(par)::value;   // parity of j
      f32x16* cur = P ? sc1 : sc0;
      f32x16* nx = P ? sc0 : sc1;
      // Copies of K(j+2) and V(j+1) of this segment. Paged: here. Contiguous:
      // between the score products of this step (or here, for a wave without
      // rows in the current tile), from buffer resources that cover the
      // tile's rows up to the sequence's last key. Rows past it, and the
      // whole tile when the segment has no such step, copy as zeros: keys
      // past the last one are masked, and a slot filled past the segment's
      // end is not read before the next segment's first copies refill it.
      StepCopies cp{};
      if constexpr (PAGED) {
        // resources built from ids loaded one step earlier; a copy the
        // segment does not have gets a resource over no rows
        const int id_k = __builtin_amdgcn_readfirstlane(raw_k);
        cp.kt = j + 2 < nt ? page_rsrc(kbase, id_k, tcur + 2 * dt) : buffer_rsrc(kbase, 0u);
        cp.vt = j + 1 < nt ? page_rsrc(vbase, id_v, tcur + dt) : buffer_rsrc(vbase, 0u);
        cp.kl = sbase + P * kSlotBytes;
        cp.vl = sbase + (3 - P) * kSlotBytes;
        id_v = id_k;
        if (j + 3 < nt) raw_k = fetch_id(tcur + 3 * dt);
      } else {
        // a copy the segment does not have gets a resource over no rows
        const uint32_t kb = j + 2 < nt ? (j + 2 == j_rag ? rag_bytes : full_bytes) : 0u;
        const uint32_t vb = j + 1 < nt ? (j + 1 == j_rag ? rag_bytes : full_bytes) : 0u;
        cp.kt = buffer_rsrc(kb2 + toff, kb);
        cp.vt = buffer_rsrc(vb1 + toff, vb);
        cp.kl = sbase + P * kSlotBytes;
        cp.vl = sbase + (3 - P) * kSlotBytes;
        toff += dstep_b;
      }
      // first key of this step's tile; whether this wave has rows that see
      // the next step's tile
      const int k0 = tcur * kBC;
      const bool nx_ok = j + 1 < nt && (tcur + dt) * kBC <= wave_last;
      tcur += dt;
      constexpr uint32_t kl = 1 - P;   // K slot of step j + 1
      constexpr uint32_t vl = 2 + P;   // V slot of step j
      if (cur_ok) {
        if (k0 > mask_k0) {
          const int rel = lim_row - k0 - 4 * khi;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * kb + 8 * (i >> 2) + (i & 3) > rel) cur[kb][i] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, cur[kb][i]);
        mx = max_xor32(mx);
        // Thresholded running max: the reference m_run moves to the new row
        // max (and the accumulators are rescaled by 2^(m2_old - m2_new)) only
        // when some row of the wave exceeds it by more than kLazy in log2
        // units; otherwise the probabilities of this tile are taken relative
        // to the old reference, at most 2^kLazy. The result is the same
        // function (the reference cancels in acc / l and enters LSE as
        // m + ln l); O is normalised by the sum of the rounded probabilities
        // the products used, so a row dominated by one key returns that key's
        // value exactly. A row whose keys so far are all masked keeps
        // m = -inf, p = 0.
        const bool grow = (mx - m_run) * a.c > kLazy<E>;
        float m2_use = m2_run, alpha = 1.f;
        if (__any(grow)) {
          const float m_new = max_quiet(m_run, mx);
          const float m2_new = m_new * a.c;
          alpha = (m_new == m_run) ? 1.f : exp2_fast(m2_run - m2_new);
          rescale(alpha);
          m_run = m_new;
          m2_run = m2_new;
          m2_use = m2_new;
        }
        if (m_run == kNegInf) m2_use = 0.f;
        // The scores of the next tile are computed even when there is none
        // (last step of the segment; they are then never used), so that this
        // path is one straight instruction stream.
        const float2 rs = fused(kl, vl, cur, nx, m2_use, std::true_type{}, cp);
        l_run = fmaf(alpha, l_run, rs.x);
        lt_run = fmaf(alpha, lt_run, rs.y);
      } else {
#pragma unroll
        for (int x = 0; x < 2 * TileLoader<D, NW>::SPW; ++x) issue_copy(cp, x);
        if (nx_ok) scores(kl, nx);
      }
      cur_ok = nx_ok;
      // The copies of this step must be resident before the next one, and
      // every wave must be done with the slots they overwrite next. Each wave
      // waits for its own copies (issued from inline assembly, so the
      // compiler does not track them), then all waves meet.
      __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      ++g;
    };
    int j = 0;
    for (; j + 1 < nt; j += 2) {
      step(Parity<0>{}, j);
      step(Parity<1>{}, j + 1);
    }
    if (j < nt) step(Parity<0>{}, j);

    const float l_tot = sum_xor32(l_run);
    const float lt_tot = sum_xor32(lt_run);
    float inv = lt_tot > 0.f ? 1.f / lt_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m2_run + log2f(l_tot)) * kLn2 : kNegInf;
    // a bad page seen by any wave spoils the tiles every wave used
    if constexpr (PAGED) bad_page = __syncthreads_or(bad_page);
    if (PAGED && (bad || bad_page)) {
      inv = __builtin_nanf("");
      lse_v = __builtin_nanf("");
    }
    // This lane's query row and head again (dense layout: from an opaque copy
    // of the lane index; kept from the segment's start they would hold
    // registers, and spill, through the key loop).
    int lane_r = lane;
    if constexpr (!PAGED) __asm__ volatile("" : "+v"(lane_r));
    const int prow_e = qw0 + (lane_r & 31);
    const int qrow_e = prow_e / G;
    const int h_e = hk * G + (prow_e - qrow_e * G);
    if (partial) {   // key split: fp32 partial (o, lse) of this split
      if (qrow_e < Nq) {
        const int64_t pr = ((q_row0 + qrow_e) * a.H + h_e) * S + split;
        float* prow = a.part_o + pr * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            store4(prow + 32 * db + 8 * gg + 4 * khi, acc[db][4 * gg] * inv,
                   acc[db][4 * gg + 1] * inv, acc[db][4 * gg + 2] * inv,
                   acc[db][4 * gg + 3] * inv);
        if (lane < 32) a.part_lse[pr] = lse_v;
      }
    } else {
      if constexpr (kStageO) {
        // The wave's O rows, rounded to the output type, into its LDS tile
        // (16-byte chunks of a row permuted by an XOR with the row), then
        // stored 16 contiguous bytes per lane: each store instruction
        // writes four whole 2*D-byte rows.
        constexpr int CPO = D / 8;   // 16-byte chunks per row
        OutT* stile = reinterpret_cast<OutT*>(&ostage[0]) + wave * (kQPW * D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int ch = 4 * db + gg;
            store4(stile + kr * D + ((ch ^ (kr % CPO)) * 8) + 4 * khi, acc[db][4 * gg] * inv,
                   acc[db][4 * gg + 1] * inv, acc[db][4 * gg + 2] * inv,
                   acc[db][4 * gg + 3] * inv);
          }
        // The store addresses depend on the lane only; computing them from an
        // opaque copy of it keeps the compiler from hoisting them out of the
        // key loop, where they would occupy registers (and spill) throughout.
        int lane_e = lane;
        __asm__ volatile("" : "+v"(lane_e));
#pragma unroll
        for (int j = 0; j < kQPW * CPO / 64; ++j) {
          const int idx = j * 64 + lane_e;
          const int row = idx / CPO, c = idx % CPO;
          const int prow2 = qw0 + row;
          const int qrow2 = prow2 / G;
          const int h2 = hk * G + (prow2 - qrow2 * G);
          const uint4 v = *reinterpret_cast<const uint4*>(stile + row * D + ((c ^ (row % CPO)) * 8));
          typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
          if (qrow2 < Nq)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v),
                reinterpret_cast<u32x4_t*>(static_cast<OutT*>(a.o) + (q_row0 + qrow2) * q_rs +
                                           static_cast<int64_t>(h2) * D + 8 * c));
        }
      } else if (qrow_e < Nq) {
        OutT* orow = static_cast<OutT*>(a.o) + (q_row0 + qrow_e) * q_rs +
                     static_cast<int64_t>(h_e) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            store4(orow + 32 * db + 8 * gg + 4 * khi, acc[db][4 * gg] * inv,
                   acc[db][4 * gg + 1] * inv, acc[db][4 * gg + 2] * inv,
                   acc[db][4 * gg + 3] * inv);
      }
      // LSE layout: [B, H, Nq] dense; [total_q, H] for ragged queries.
      const int64_t li = PAGED ? (q_row0 + qrow_e) * a.H + h_e
                               : (static_cast<int64_t>(b) * a.H + h_e) * Nq + qrow_e;
      if (lane < 32 && qrow_e < Nq) a.lse[li] = lse_v;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: 32x32x2 fp32 matrix-core ops, probabilities kept in fp32.
// ---------------------------------------------------------------------------
template <int D>
struct PolicyF32 {
  using In = float;
  static constexpr int KS = D + 1;     // odd stride: column reads hit 32 distinct banks
  static constexpr int VS = D + 4;
  static constexpr int K_ELEMS = kBC * KS;
  static constexpr int V_ELEMS = kBC * VS;
  static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 4;
  static constexpr int CPR = D / 4;
  static constexpr int PER_THREAD = kBC * CPR / kThreads;
  static constexpr int QF = D / 2;
  static_assert(PER_THREAD * kThreads == kBC * CPR, "tile must split evenly");

  float qf[QF];   // Q[row][c + (D/2)(l/32)]
  float4 kst[PER_THREAD];
  float4 vst[PER_THREAD];

  __device__ __forceinline__ void load_q(const In* qrow, bool valid, int lane) {
    const In* p = qrow + (D / 2) * (lane >> 5);
#pragma unroll
    for (int c = 0; c < QF; c += 4) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (valid) u = *reinterpret_cast<const float4*>(p + c);
      qf[c] = u.x; qf[c + 1] = u.y; qf[c + 2] = u.z; qf[c + 3] = u.w;
    }
  }

  __device__ __forceinline__ void stage_load(const In* kb, const In* vb, int64_t rs, int k0,
                                             int nk, int tid) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = tid + r * kThreads;
      const int key = k0 + ci / CPR, dc = ci % CPR;
      float4 ku = make_float4(0.f, 0.f, 0.f, 0.f), vu = ku;
      if (key < nk) {
        ku = *reinterpret_cast<const float4*>(kb + key * rs + dc * 4);
        vu = *reinterpret_cast<const float4*>(vb + key * rs + dc * 4);
      }
      kst[r] = ku;
      vst[r] = vu;
    }
  }

  __device__ __forceinline__ void stage_store(unsigned char* buf, int tid) {
    In* kl = reinterpret_cast<In*>(buf);
    In* vl = kl + K_ELEMS;
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = tid + r * kThreads;
      const int key = ci / CPR, dc = ci % CPR;
      In* kp = kl + key * KS + dc * 4;
      kp[0] = kst[r].x; kp[1] = kst[r].y; kp[2] = kst[r].z; kp[3] = kst[r].w;
      *reinterpret_cast<float4*>(vl + key * VS + dc * 4) = vst[r];
    }
  }

  __device__ __forceinline__ void scores(const unsigned char* buf, int lane, f32x16 s[2]) const {
    const In* kl = reinterpret_cast<const In*>(buf);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = {};
      const In* row = kl + (32 * kb + (lane & 31)) * KS + (D / 2) * (lane >> 5);
#pragma unroll
      for (int c = 0; c < QF; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(row[c], qf[c], acc, 0, 0, 0);
      s[kb] = acc;
    }
  }

  // Step (kb, i) contracts over the pair of keys held in register i by the
  // two half-waves: key 32kb + 8(i/4) + i%4 (+4 for the upper half).
  __device__ __forceinline__ void pv(const unsigned char* buf, int lane, const f32x16 p[2],
                                     f32x16* acc) const {
    const In* vl = reinterpret_cast<const In*>(buf) + K_ELEMS;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + (i & 3) + 4 * (lane >> 5);
        const In* vrow = vl + key * VS + (lane & 31);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db], p[kb][i], acc[db], 0, 0, 0);
      }
    }
  }
};

template <class P, typename OutT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const FwdParams a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * P::BUF_BYTES];
  using In = typename P::In;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int L = xcd_remap(static_cast<int>(blockIdx.x), a.total);
  const int bh = L / a.n_qblocks;
  int qb = L - bh * a.n_qblocks;
  if (CAUSAL) qb = a.n_qblocks - 1 - qb;   // longest causal rows first within each head
  const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;
  const int q0 = qb * kBR;
  const int qw0 = q0 + wave * kQPW;
  const int qrow = qw0 + (lane & 31);

  const int64_t q_rs = static_cast<int64_t>(a.H) * D;
  const int64_t kv_rs = static_cast<int64_t>(a.Hkv) * D;
  const In* kbase = static_cast<const In*>(a.k) + static_cast<int64_t>(b) * a.Nk * kv_rs +
                    static_cast<int64_t>(hk) * D;
  const In* vbase = static_cast<const In*>(a.v) + static_cast<int64_t>(b) * a.Nk * kv_rs +
                    static_cast<int64_t>(hk) * D;

  P pol;
  pol.load_q(static_cast<const In*>(a.q) + (static_cast<int64_t>(b) * a.Nq + qrow) * q_rs +
                 static_cast<int64_t>(h) * D,
             qrow < a.Nq, lane);

  int last_key = a.Nk - 1;
  int wave_last = a.Nk - 1;
  if (CAUSAL) {
    last_key = min(last_key, q0 + kBR - 1 + a.off);
    wave_last = min(wave_last, qw0 + kQPW - 1 + a.off);
  }
  const int n_tiles = last_key >= 0 ? last_key / kBC + 1 : 0;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = kNegInf, m2_run = kNegInf, l_run = 0.f;

  if (n_tiles > 0) {
    pol.stage_load(kbase, vbase, kv_rs, 0, a.Nk, tid);
    pol.stage_store(smem, tid);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = j * kBC;
    if (j + 1 < n_tiles) pol.stage_load(kbase, vbase, kv_rs, k0 + kBC, a.Nk, tid);
    if (k0 <= wave_last) {
      const unsigned char* buf = smem + (j & 1) * P::BUF_BYTES;
      f32x16 s[2];
      pol.scores(buf, lane, s);

      const bool need_mask = (k0 + kBC > a.Nk) || (CAUSAL && k0 + kBC - 1 > qw0 + a.off);
      if (need_mask) {
        const int lim = CAUSAL ? min(a.Nk - 1, qrow + a.off) : a.Nk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (key > lim) s[kb][i] = kNegInf;
          }
      }

      // Online softmax update for this lane's query row.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m2_new = m_new * a.c;
      const float m2_use = (m_new == kNegInf) ? 0.f : m2_new;
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m2_run - m2_new);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(fmaf(s[kb][i], a.c, -m2_use));
          s[kb][i] = p;
          rs += p;
        }
      l_run = fmaf(alpha, l_run, rs);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      m_run = m_new;
      m2_run = m2_new;

      pol.pv(buf, lane, s, acc);
    }
    if (j + 1 < n_tiles) pol.stage_store(smem + ((j + 1) & 1) * P::BUF_BYTES, tid);
    __syncthreads();
  }

  // Epilogue: normalise once, store O in the output type and LSE in fp32.
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < a.Nq) {
    OutT* orow = static_cast<OutT*>(a.o) + (static_cast<int64_t>(b) * a.Nq + qrow) * q_rs +
                 static_cast<int64_t>(h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(orow + 32 * db + 8 * g + 4 * (lane >> 5), acc[db][4 * g] * inv,
               acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
    if (lane < 32)
      a.lse[(static_cast<int64_t>(b) * a.H + h) * a.Nq + qrow] =
          l_tot > 0.f ? (m2_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

template <class P, typename OutT, int D>
hipError_t launch_t(const FwdParams& p, bool causal, hipStream_t s) {
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<P, OutT, D, true>), dim3(p.total), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_kernel<P, OutT, D, false>), dim3(p.total), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

constexpr int kNW16 = 8;   // waves per workgroup of the 16-bit kernel (2 per SIMD)
// A grid of fewer 8-wave workgroups than the chip has CUs leaves CUs idle and
// runs two waves on each SIMD it uses; the same rows in 4-wave workgroups
// (128 packed rows each) spread over twice the CUs with one wave per SIMD,
// and in 2-wave workgroups (64 rows) over four times as many when even the
// 4-wave grid is short of the CU count and the 2-wave one is not over it.
constexpr int kNW16Small = 4;
constexpr int kNW16Tiny = 2;
constexpr int kCus = 256;

template <class E, typename OutT, int D, bool PAGED, int NW = kNW16>
hipError_t launch16(const FwdParams& p, bool causal, hipStream_t s) {
  if (causal)
    hipLaunchKernelGGL((fwd16_kernel<E, OutT, D, true, NW, PAGED>), dim3(p.total),
                       dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((fwd16_kernel<E, OutT, D, false, NW, PAGED>), dim3(p.total),
                       dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t dispatch_nw(const FwdParams& p, const ForwardArgs& a, hipStream_t s) {
  const bool c = a.causal != 0;
  if (a.in_dtype == FA_BF16)
    return a.out_dtype == FA_F32 ? launch16<BF16, float, D, false, NW>(p, c, s)
                                 : launch16<BF16, __bf16, D, false, NW>(p, c, s);
  return a.out_dtype == FA_F32 ? launch16<F16, float, D, false, NW>(p, c, s)
                               : launch16<F16, _Float16, D, false, NW>(p, c, s);
}

template <int D>
hipError_t dispatch_d(const FwdParams& p, const ForwardArgs& a, hipStream_t s, int nw) {
  if (a.in_dtype == FA_F32) return launch_t<PolicyF32<D>, float, D>(p, a.causal != 0, s);
  if (nw == kNW16Tiny) return dispatch_nw<D, kNW16Tiny>(p, a, s);
  return nw == kNW16Small ? dispatch_nw<D, kNW16Small>(p, a, s) : dispatch_nw<D, kNW16>(p, a, s);
}

template <int D>
hipError_t dispatch_paged_d(const FwdParams& p, const ForwardPagedArgs& a, hipStream_t s) {
  const bool c = a.causal != 0;
  if (a.dtype == FA_BF16)
    return a.out_dtype == FA_F32 ? launch16<BF16, float, D, true>(p, c, s)
                                 : launch16<BF16, __bf16, D, true>(p, c, s);
  return a.out_dtype == FA_F32 ? launch16<F16, float, D, true>(p, c, s)
                               : launch16<F16, _Float16, D, true>(p, c, s);
}

}  // namespace

hipError_t launch_forward_paged(const ForwardPagedArgs& a, hipStream_t s) {
  FwdParams p{};
  p.q = a.q; p.k = a.k_pool; p.v = a.v_pool; p.o = a.o; p.lse = a.lse;
  p.B = a.B; p.H = a.H; p.Hkv = a.Hkv;
  p.group = a.H / a.Hkv;
  const int br = kNW16 * kQPW;
  const int max_qb = static_cast<int>((int64_t{a.max_q_len} * p.group + br - 1) / br);
  const bool partial = !a.causal && a.part_o != nullptr;
  p.kv_splits = partial ? a.kv_splits : 1;
  p.units = a.causal ? (max_qb + 1) / 2 : max_qb * p.kv_splits;
  p.fixed_kv_len = a.fixed_kv_len;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.total = (a.B * a.Hkv + kXcds - 1) / kXcds * kXcds * p.units;
  p.c = a.scale * kLog2e;
  p.qo_indptr = a.qo_indptr;
  p.kv_lens = a.kv_lens;
  p.block_table = a.block_table;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.total_q = a.total_q;
  p.max_q_len = a.max_q_len;
  if (p.total == 0) return hipSuccess;
  // Sequences with a single query row (decode tokens in a mixed batch) go
  // through the split-KV decode kernel's page streaming instead: here such a
  // row would keep a whole workgroup of 8 waves waiting on every key tile
  // for the work of one wave.
  p.skip_single = !partial && a.qo_indptr && a.kv_lens && p.group <= 16 && a.max_q_len >= 1;
  if (p.skip_single) {
    const hipError_t e = launch_decode_rows(a, s);
    if (e != hipSuccess) return e;
  }
  return a.d == 64 ? dispatch_paged_d<64>(p, a, s) : dispatch_paged_d<128>(p, a, s);
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s) {
  FwdParams p{};
  int nw = 0;
  p.kv_splits = 1;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
  p.B = a.B; p.H = a.H; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
  p.group = a.H / a.Hkv;
  const bool f32 = a.in_dtype == FA_F32;
  if (f32) {   // one workgroup per (batch, head, 128-row query block)
    p.n_qblocks = (a.Nq + kBR - 1) / kBR;
    p.units = p.n_qblocks;
    p.total = a.B * a.H * p.units;
  } else {     // per (batch, KV head): blocks of packed (query, head) rows
    auto blocks = [&](int nw) {
      const int br = nw * kQPW;
      p.n_qblocks = static_cast<int>((int64_t{a.Nq} * p.group + br - 1) / br);
      // causal: query blocks u and n-1-u share one workgroup
      p.units = a.causal ? (p.n_qblocks + 1) / 2 : p.n_qblocks;
      return int64_t{a.B} * a.Hkv * p.units;   // workgroups with work
    };
    nw = kNW16;
    if (blocks(kNW16) < kCus) {
      nw = kNW16Small;
      // 2-wave workgroups only while each still gets a CU of its own: two
      // sharing a CU take twice as long as one 4-wave workgroup of theirs
      if (blocks(kNW16Small) < kCus && blocks(kNW16Tiny) <= kCus)
        nw = kNW16Tiny;
      else
        blocks(kNW16Small);
    }
    p.total = (a.B * a.Hkv + kXcds - 1) / kXcds * kXcds * p.units;
  }
  p.c = a.scale * kLog2e;
  p.off = a.Nk - a.Nq;
  if (p.total == 0) return hipSuccess;
  return a.d == 64 ? dispatch_d<64>(p, a, s, nw) : dispatch_d<128>(p, a, s, nw);
}

}  // namespace fa
