// Pieces shared by the attention kernels (attention_fwd.hip: forward;
// attention.hip: backward): tile shapes, LDS layouts and fragment reads, and
// the cutting of long causal rows into chunks.  See attention.hip for what
// the kernels compute.
#pragma once

#include <math.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace ptb {
namespace {

constexpr int BQ = 128;   // queries per workgroup (forward, dQ): 4 waves x 32
constexpr int BKV = 64;   // keys per LDS tile (forward, dQ)
constexpr int BKB = 128;  // keys per workgroup (dK/dV): 4 waves x 32
constexpr int BQB = 64;   // queries per LDS tile (dK/dV)

// Rows of D bf16 in LDS, addressed in 16-byte chunks: chunk c of row r sits
// at chunk slot c ^ rowswz<D>(r).  The LDS serves 64 banks of 4 bytes; a
// 16-byte read is served 16 lanes at a time, an 8-byte read (plain or
// transposing) 32 lanes at a time.  The swizzle keeps both fragment reads
// below free of bank conflicts:
//   D = 128 (256-byte rows, each spanning every bank): the two 2-bit fields
//     of r & 15 trade places, so 16 aligned consecutive rows read at one
//     chunk take 16 distinct slots, and the 4 aligned rows x 4 aligned chunks
//     of 32 lanes of a transposing read take 4 distinct groups of 4 slots;
//   D = 64 (128-byte rows, the row's parity picking half of the banks): rows
//     of one parity among 16 aligned rows take 8 distinct slots, and rows
//     4a + p and 4a + 2 + p take different halves of the row.
template <int D>
__device__ __forceinline__ int rowswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ u16* row_chunk(u16* base, int r, int c) {
  return base + r * D + ((c ^ rowswz<D>(r)) << 3);
}
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const u16* base, int r, int c) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(base + r * D + ((c ^ rowswz<D>(r)) << 3)));
}

// perm16 swaps rows 4..7 and 8..11 inside every 16 (see the DMA-staged
// tiles below).
__device__ __forceinline__ int perm16(int r) {
  const int p = r & 15;
  return (r & ~15) | ((p >= 4 && p < 12) ? (p ^ 12) : p);
}

// MFMA A operand of the transpose of a row tile [R][D] (rows swizzled by
// rowswz<D>) over columns [rb, rb + 32) and the 16 tile rows of step ks, the
// rows taken in perm16 order (the order in which a packed 32 x 32 accumulator
// runs over them): lane l gets X^T[rb + l % 32][perm16(16 ks + 8 (l / 32) ..
// +7)].  Each 16-lane group reads 4 rows x 16 columns (4 u16 per lane, 8
// bytes inside one 16-byte chunk), transposed by ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ bf16x8 frag_rows_tr(const u16* tile, int rb, int ks, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int m = rb + 16 * (q & 1) + 4 * (j & 3);
  v4s h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int kk = ks * 16 + 8 * (q >> 1) + 4 * hh + (j >> 2);
    const int r = perm16(kk);
    h[hh] = lds_read_tr16(tile + r * D + (((m >> 3) ^ rowswz<D>(r)) << 3) + (m & 7));
  }
  uint4 u;
  u.x = static_cast<uint16_t>(h[0][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[0][1])) << 16);
  u.y = static_cast<uint16_t>(h[0][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[0][3])) << 16);
  u.z = static_cast<uint16_t>(h[1][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[1][1])) << 16);
  u.w = static_cast<uint16_t>(h[1][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[1][3])) << 16);
  return as_bf16x8(u);
}

// Eight accumulator values as fp16 (round to nearest even, no saturation:
// the attention's dS values stay far inside the fp16 range).
__device__ __forceinline__ uint32_t pack2h_pk(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
}
__device__ __forceinline__ bf16x8 pack8h(const f32x16& a, int base) {
  return as_bf16x8(make_uint4(pack2h_pk(a[base + 0], a[base + 1]), pack2h_pk(a[base + 2], a[base + 3]),
                              pack2h_pk(a[base + 4], a[base + 5]), pack2h_pk(a[base + 6], a[base + 7])));
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
  return as_bf16x8(make_uint4(pack2bf_pk(a[base + 0], a[base + 1]), pack2bf_pk(a[base + 2], a[base + 3]),
                              pack2bf_pk(a[base + 4], a[base + 5]), pack2bf_pk(a[base + 6], a[base + 7])));
}

// ------------------------------------------------- DMA-staged tiles
// A tile of R rows (keys or queries) x D columns goes from HBM to LDS by DMA
// (buffer_load ... lds, 64 lanes x 16 bytes = 1 KB per load), in one of two
// layouts:
//   rows  (OUTER = false): [R][D], rows of 2D bytes, 16-byte chunk c of row r
//         at slot c ^ rowswz<D>(r); MFMA fragments by row_frag;
//   outer (OUTER = true):  [D / 64][R][64], row rho of a 64-column block
//         holding tile row perm16(rho), chunk c at slot c ^ oswz(rho);
//         fragments of the transpose by frag_outer<R>.
// perm16 swaps rows 4..7 and 8..11 inside every 16.  A 32 x 32 MFMA
// accumulator holds, per lane and 16-row step, rows 4g..4g+3 and 8+4g..8+4g+3
// (g = lane / 32); packed as the B operand of a second product it therefore
// runs over the rows in perm16 order, and the outer tile's rows are stored in
// that order so that both operands agree.  The source row of each lane applies
// the swizzle and the permutation; rows at or beyond the operand's end read
// as zeros (buffer range check).


template <int D, int R, bool OUTER>
struct TileDma {
  static constexpr int NL = R * D * 2 / 1024;  // loads per tile
  static constexpr int LPW = NL / 4;            // ... per wave
  static_assert(LPW >= 1 && NL % 4 == 0, "tile too small for four waves");
  i32x4 desc;
  int off[LPW];  // per-lane byte offsets at tile row 0
  int ld;

  // rows of the operand at base + row * ld_ (elements), nrows of them
  __device__ __forceinline__ void init(const u16* base, int ld_, int nrows, int wave, int lane) {
    ld = ld_;
    desc = make_desc(base, static_cast<uint32_t>(((nrows - 1) * ld + D) * 2));
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int inst = wave * LPW + i;
      if constexpr (!OUTER) {
        constexpr int CPR = 2 * D / 16;  // chunks per row
        const int r = inst * (64 / CPR) + lane / CPR;
        const int c = (lane % CPR) ^ rowswz<D>(r);
        off[i] = (r * ld + c * 8) * 2;
      } else {
        constexpr int LPB = R / 8;  // loads per 64-column block
        const int blk = inst / LPB, rho = (inst % LPB) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ oswz(rho);
        off[i] = (perm16(rho) * ld + blk * 64 + c * 8) * 2;
      }
    }
  }
  // tile rows row0 .. row0 + R - 1 into LDS bytes [lds, lds + 2 R D)
  __device__ __forceinline__ void issue(uint32_t lds, int row0, int wave) const {
    const int soff = row0 * ld * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) lds_dma16(desc, lds + (wave * LPW + i) * 1024, off[i], soff);
  }
  // load i (0..LPW-1) of issue, or of issue_none (valid false), alone
  __device__ __forceinline__ void issue_one(uint32_t lds, int row0, int wave, int i, bool valid) const {
    lds_dma16(desc, lds + (wave * LPW + i) * 1024, off[i], valid ? row0 * ld * 2 : kOutOfRange);
  }
  // the same loads with an offset beyond any operand: they return zeros
  // without touching memory (zeros land in [lds, lds + 2 R D)), so that a
  // wave's count of loads in flight stays the same past the last tile
  __device__ __forceinline__ void issue_none(uint32_t lds, int wave) const {
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      lds_dma16(desc, lds + (wave * LPW + i) * 1024, off[i], kOutOfRange);
  }
};

// ------------------------------------------------------- row splitting
// A "row" is one 128-wide block of queries (forward, dQ) or keys (dK/dV);
// it walks tiles of 64 along the other axis.  Under a causal mask the rows
// carry very different amounts of work, so long rows are cut into chunks of
// at most `ch` tiles, one workgroup each; the chunks of a row are combined by
// the last of them to finish (fp32 partials at device scope, an arrival
// counter per row).  Rows are taken longest first.
struct RowSpan {
  int begin, end;  // [begin, end) along the tiled axis
};
__host__ __device__ inline RowSpan query_row(int qt, int s, int window) {
  const int q0 = qt * BQ;
  RowSpan r;
  r.begin = (q0 - window + 1 > 0 ? q0 - window + 1 : 0) & ~(BKV - 1);
  r.end = q0 + BQ < s ? q0 + BQ : s;
  return r;
}
__host__ __device__ inline RowSpan key_row(int kt, int s, int window) {
  const int k0 = kt * BKB;
  RowSpan r;
  r.begin = k0 & ~(BQB - 1);
  const long e = static_cast<long>(k0) + BKB - 1 + window;
  r.end = e < s ? static_cast<int>(e) : s;
  return r;
}
__host__ __device__ inline int row_tiles(RowSpan r) { return (r.end - r.begin + 63) / 64; }
__host__ __device__ inline int row_chunks(RowSpan r, int ch) {
  const int nt = row_tiles(r);
  return nt <= 0 ? 1 : (nt + ch - 1) / ch;
}

// The work item of workgroup x within one (batch, head): its row, chunk,
// span, the row's chunk count, and (for split rows) its partial slot.
struct RowItem {
  int row, chunk, nchunks, slot;
  RowSpan span;
};
template <bool QUERY_ROWS>
__device__ __forceinline__ RowItem decode_row_item(int x, int nrows, int s, int window, int ch) {
  RowItem it{};
  int slot = 0;
  for (int i = 0; i < nrows; ++i) {
    const int row = QUERY_ROWS ? nrows - 1 - i : i;  // longest rows first
    const RowSpan sp = QUERY_ROWS ? query_row(row, s, window) : key_row(row, s, window);
    const int nch = row_chunks(sp, ch);
    if (x < nch) {
      it.row = row;
      it.chunk = x;
      it.nchunks = nch;
      it.slot = slot + x;
      it.span.begin = sp.begin + x * ch * 64;
      const int e = sp.begin + (x + 1) * ch * 64;
      it.span.end = e < sp.end ? e : sp.end;
      return it;
    }
    x -= nch;
    if (nch > 1) slot += nch;
  }
  it.nchunks = 0;  // past the last item (not launched)
  return it;
}

// fp32 store and load at device (agent) scope: coherent across the XCDs
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A lane's 16 fp32 values of a 1024-float block of a split row's partial, at
// device scope in 16-byte accesses: the cache policy of relaxed agent-scope
// atomics (sc1) on buffer loads and stores.  Value e of lane l sits at float
// [e / 4][l][e % 4] of the block, so one access covers 1 KB.  `blk` is the
// block's first float in the slot that `r` covers (below 2^29 floats).
constexpr int kDevPolicy = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(float* slot, int floats) {
  return __builtin_amdgcn_make_buffer_rsrc(slot, static_cast<short>(0), floats * 4, 0x00020000);
}
template <typename V>
__device__ __forceinline__ void st16_dev(__amdgpu_buffer_rsrc_t r, int blk, int lane, const V& v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned d0 = __float_as_uint(v[4 * q]), d1 = __float_as_uint(v[4 * q + 1]);
    const unsigned d2 = __float_as_uint(v[4 * q + 2]), d3 = __float_as_uint(v[4 * q + 3]);
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    const u4v d = {d0, d1, d2, d3};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, (blk + q * 256 + lane * 4) * 4, 0, kDevPolicy);
  }
}
__device__ __forceinline__ void ld16_dev(__amdgpu_buffer_rsrc_t r, int blk, int lane, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto d = __builtin_amdgcn_raw_buffer_load_b128(r, (blk + q * 256 + lane * 4) * 4, 0,
                                                         kDevPolicy);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[4 * q + k] = __uint_as_float(d[k]);
  }
}

// Scratch of the split rows of one launch.
struct RowSplit {
  float* partials;  // slot-major; `per_slot` floats each
  int* counters;    // one per (batch, head, row): zero on entry, left zero
  int ch;           // tiles per chunk
  int split_slots;  // partial slots per (batch, head)
  int nb;           // batches x heads
};

// The item, head and batch of this workgroup.  The grid is one-dimensional,
// (batch, head) fastest and then the item, so that the hardware, which hands
// out workgroups in index order, starts every head's longest items before any
// head's shorter ones (items are numbered longest first within a head).
struct RowBlock {
  int item, hd, bi;
};
__device__ __forceinline__ RowBlock row_block(const RowSplit& rs, int n) {
  const int x = static_cast<int>(blockIdx.x);
  const int hb = x % rs.nb;
  RowBlock r;
  r.item = x / rs.nb;
  r.hd = hb % n;
  r.bi = hb / n;
  return r;
}

// Chunk length for the rows of one launch, chosen on a model of the
// dispatch.  The hardware hands out workgroups in grid order (row_block) to
// `slots` places at a time (workgroups per CU x CUs), each to the first place
// that frees up.  An item costs its 64-wide tiles plus a fixed start (loading
// its own rows, filling the ring); a chunk of a split row also stores its
// partial, and the last chunk of a row merges them.  The candidates are the
// lengths at which the longest row's chunk count changes; the one with the
// earliest simulated finish wins (the longer on ties: fewer partials), among
// those whose partials fit the scratch.  `tile_cost` scales every cost (a
// kernel build whose tiles take longer), `finish` receives the simulated
// finish in those units.  The choice is kept per thread for the last few
// shapes asked (the simulation is the costly part).
struct RowPlanKey {
  int b, s, n, window, nrows, per_slot, slots, max_counters;
  size_t partial_floats;
  double tile_cost;
  bool operator==(const RowPlanKey& o) const {
    return b == o.b && s == o.s && n == o.n && window == o.window && nrows == o.nrows &&
           per_slot == o.per_slot && slots == o.slots && max_counters == o.max_counters &&
           partial_floats == o.partial_floats && tile_cost == o.tile_cost;
  }
};
struct RowPlanEntry {
  RowPlanKey key;
  long ch;
  double finish;
};

// Places for workgroups of `kernel` (256 threads) on the device: workgroups
// per CU as the compiler's resource use allows, times the CUs.
template <typename K>
int launch_slots(K kernel, const AttnScratch& sc) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu * (sc.cus > 0 ? sc.cus : 256);
}

template <bool QUERY_ROWS>
hipError_t plan_rows(int b, int s, int n, int window, int nrows, int per_slot, int slots,
                     const AttnScratch& sc, RowSplit* rs, int* items_per_head,
                     double tile_cost = 1.0, double* finish = nullptr) {
  const long nb = static_cast<long>(b) * n;
  if (nb <= 0 || nrows <= 0 || slots <= 0) return hipErrorInvalidValue;
  // rows in item order (decode_row_item): longest first
  std::vector<int> tiles(nrows);
  int tmax = 1;
  for (int i = 0; i < nrows; ++i) {
    const int row = QUERY_ROWS ? nrows - 1 - i : i;
    tiles[i] = row_tiles(QUERY_ROWS ? query_row(row, s, window) : key_row(row, s, window));
    tmax = std::max(tmax, tiles[i]);
  }
  auto chunks = [](int nt, long ch) { return nt <= 0 ? 1L : (nt + ch - 1) / ch; };
  auto fits = [&](long ch, long* items_out) {
    long items = 0, split = 0;
    for (int nt : tiles) {
      const long nc = chunks(nt, ch);
      items += nc;
      if (nc > 1) split += nc;
    }
    *items_out = items;
    return (split == 0 || (split * nb * per_slot <= static_cast<long>(sc.partial_floats) &&
                           nb * nrows <= sc.max_counters)) &&
           items * nb < (1L << 31);
  };
  // partial store and merge, in tiles, scaled from the forward's measured
  // costs (64 KB partials: 0.7 and 0.4 per chunk)
  const double pscale = per_slot / (128.0 * 128.0 + 512.0);
  auto simulate = [&](long ch) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
    double end = 0.0;
    for (int i = 0; i < nrows; ++i) {
      const long nc = chunks(tiles[i], ch);
      for (long x = 0; x < nc; ++x) {
        const long t = std::min<long>(ch, tiles[i] - x * ch);
        double cost = 2.3 + static_cast<double>(std::max<long>(t, 0));
        if (nc > 1) cost += 0.7 * pscale + (x == nc - 1 ? 0.4 * pscale * nc : 0.0);
        cost *= tile_cost;
        for (long h = 0; h < nb; ++h) {
          double t0 = 0.0;
          if (static_cast<long>(free_at.size()) >= slots) {
            t0 = free_at.top();
            free_at.pop();
          }
          free_at.push(t0 + cost);
          end = std::max(end, t0 + cost);
        }
      }
    }
    return end;
  };
  const RowPlanKey key{b,  s, n, window, nrows, per_slot, slots, sc.max_counters, sc.partial_floats,
                       tile_cost};
  constexpr int kCache = 4;
  thread_local RowPlanEntry cache[kCache] = {};
  thread_local int next_slot = 0;
  long best = 0;
  double best_t = 0.0;
  const RowPlanEntry* hit = nullptr;
  for (const RowPlanEntry& c : cache)
    if (c.ch > 0 && c.key == key) hit = &c;
  if (hit != nullptr) {
    best = hit->ch;
    best_t = hit->finish;
  } else {
    long prev = -1, items = 0;
    for (int k = 1; k <= tmax && k <= 64; ++k) {
      const long ch = (tmax + k - 1) / k;
      if (ch == prev) continue;
      prev = ch;
      if (!fits(ch, &items)) continue;
      // beyond this many workgroups the simulation costs more than it saves
      if (items * nb > 200000 && best > 0) break;
      const double t = simulate(ch);
      if (best == 0 || t < best_t - 1e-9) {
        best = ch;
        best_t = t;
      }
    }
    // nothing fits: chunks grow until the partials do
    for (long ch = tmax; best == 0; ch *= 2) {
      if (fits(ch, &items)) {
        best = ch;
        best_t = simulate(ch);
      }
      if (ch > (1L << 20)) return hipErrorInvalidValue;
    }
    cache[next_slot] = RowPlanEntry{key, best, best_t};
    next_slot = (next_slot + 1) % kCache;
  }
  if (finish != nullptr) *finish = best_t;
  long items = 0, split = 0;
  for (int nt : tiles) {
    const long nc = chunks(nt, best);
    items += nc;
    if (nc > 1) split += nc;
  }
  rs->partials = sc.partials;
  rs->counters = sc.counters;
  rs->ch = static_cast<int>(best);
  rs->split_slots = static_cast<int>(split);
  rs->nb = static_cast<int>(nb);
  *items_per_head = static_cast<int>(items);
  return hipSuccess;
}

}  // namespace
}  // namespace ptb
