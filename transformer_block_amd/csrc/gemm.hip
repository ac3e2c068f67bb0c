// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16): persistent
// kernel, operands streamed from global memory straight into LDS, fused
// epilogues.
//
// One kernel template covers the six matrix products of the Parallel
// Transformer Block layer (MegaScale reading notes, section 1.1, eq (4); fused
// QKV projection, section 1.3; MLP Y = GeLU(XA)B, Megatron-LM tensor-parallel
// explainer, section 2.1):
//   forward   [QKV | FC1]:  a [T,h]      x [W_qkv | W_fc1]      -> qkv, u, GeLU(u)
//             [O ; FC2]:    [c | g]      x [W_o ; W_fc2]  + x   -> y
//   backward  dgrad:        dy x [W_o ; W_fc2]^T  (x GeLU'(u))  -> dc, du
//                           dZ x [W_qkv | W_fc1]^T              -> da
//             wgrad:        [c | g]^T x dy                      -> dW_o, dW_fc2
//                           a^T x dZ                            -> dW_qkv, dW_fc1
// Concatenations are addressed in place (two-segment operands), never copied.
//
// Tiling.  A 256-thread workgroup (4 waves of 64 lanes, 2 x 2, 128 x 128 of C
// per wave) owns 256 x 256 tiles of C and walks K in steps of 64.  Operand
// tiles go from global memory to LDS by buffer_load ... lds (16 bytes per lane,
// no trip through registers, whole 128-byte lines) into two stages of 64 KB,
// one k-step ahead of the matrix cores.  Operands stored k-contiguous sit in
// LDS as rows of 64 k-values and feed the MFMAs with one ds_read_b128 per
// fragment; operands stored outer-contiguous sit as [64-column block][64 k]
// [64 columns] and are transposed by the LDS read itself (ds_read_b64_tr_b16).
// Both layouts are XOR-swizzled so that the fragment reads are free of bank
// conflicts.
//
// Scheduling.  The grid is persistent: one workgroup per CU.  Output tiles
// are work items handed out in rounds (item i to workgroup i mod G), so the
// items of a round run side by side at the same k positions and share their
// operand panels in L2.  When the tiles do not fill the last round, its items
// are cut along k into pieces that do; a tile made of several pieces is
// summed, in a fixed order, by whichever piece finishes last (an arrival
// counter per tile and fp32 partial tiles written at device scope), so no
// workgroup ever waits on another.  Two grouped products whose K differ by a
// whole factor are cut into pieces of equal length first.  Workgroup ids are
// remapped so that each XCD (each with its own L2) takes a contiguous run of
// items in every round.
//
// FP8.  The same eight-wave kernel multiplies 8-bit operands (E4M3 or E5M2,
// Megatron-LM tuning post, mixed-precision section) with
// v_mfma_f32_32x32x64_f8f6f4.  Both operands are then k-contiguous and a
// 128-byte LDS row holds 128 k-values instead of 64, so the DMA, the swizzle
// and the fragment reads are the bf16 ones byte for byte; one FP8 MFMA takes
// the 32 bytes that two consecutive bf16 k-steps would (A and B see the same
// k order, so the sum is the product).  The epilogue first multiplies the
// fp32 sums by the dequantization factor 1/(sA sB) of the operands' current
// scales, sX = FMAX / amax(X), which it derives from the amax values the
// cast kernels left in device memory.  With block (MX) scales the matrix
// cores apply the scales themselves (v_mfma_scale_f32_32x32x64_f8f6f4): the
// loader waves bring each stage tile's scale words (one 32-bit word per row
// and 128-wide k-step) into a small LDS ring beside the operand ring, and
// each lane passes the byte of its row's 32-wide k-block.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace ptb {
namespace {

constexpr int TILE = 256;                  // BM = BN
constexpr int BK = 64;                     // k per pipeline stage
constexpr int NSTAGE = 2;
constexpr int STAGE = 2 * TILE * BK;       // u16 elements: A tile, then B tile (64 KB)
constexpr int EPI_LD = 36;                 // fp32 row stride of the epilogue staging
constexpr int GM = 8;                      // tile rows per L2 group
constexpr int WAVES = 8;                   // 2 per SIMD: 2 (rows) x 4 (columns)
constexpr int LOADERS = 4;                 // waves 0-3 issue every DMA load
constexpr int WM = 128, WN = 64;           // outputs per wave
constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 MFMA blocks per wave
constexpr int PARTIAL_FLOATS = TILE * TILE;

// k-contiguous stage tile [256 rows][64 k]: 128-byte rows, 16-byte chunk c of
// row r at chunk slot c ^ kswz(r).  The 16 rows of one ds_read_b128 pass hit
// 16 distinct 16-byte bank groups, and the swizzle of a 1 KB load (8 rows)
// depends on the load only through its parity.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }

// The DMA of one operand's stage tile: 32 KB = 32 loads of 1 KB, eight per
// loader wave, each a run of whole 128-byte lines.  Load i of loader wave w
// (inst = 8w + i)
// fills LDS bytes [1 KB * inst, +1 KB):
//   k-contiguous:     rows 8*inst .. +7, all 64 k;
//   outer-contiguous: k-rows 8*(inst%8) .. +7 of outer block inst/8 (64 wide).
// A wave's eight loads cover one aligned block of 64 outer indices, so with
// split points at multiples of 64 the segment of an outer split is uniform
// per wave; the segment of a k-split follows k0.
template <int MAJ>
struct StageLoader {
  // Per-lane byte offset of the lane's 16 bytes at k = 0: offA while k is in
  // segment 0 of a k-split operand, offB in segment 1; for an outer split
  // both hold the offset in the wave's segment.
  int offA[8], offB[8];
  i32x4 dA, dB;  // buffer resources matching offA and offB
  int ldA, ldB;  // leading dimensions (the k stride of outer-contiguous tiles) likewise
  // the operand's shape, held in registers: the loads are inline assembly
  // with a memory clobber, after which fields read from memory would be
  // loaded again (and every scalar load waits on the LDS counter too)
  int ld0, ld1, split, split_on_k;

  __device__ __forceinline__ void init(const Operand& op, int r0, int wave, int lane) {
    ld0 = __builtin_amdgcn_readfirstlane(op.ld0);
    ld1 = __builtin_amdgcn_readfirstlane(op.ld1);
    split = __builtin_amdgcn_readfirstlane(op.split);
    split_on_k = __builtin_amdgcn_readfirstlane(op.split_on_k);
    const int wseg = (!split_on_k && r0 + 64 * wave >= split) ? 1 : 0;
    const i32x4 d0 = make_desc(op.p0, op.bytes0), d1 = make_desc(op.p1, op.bytes1);
    dA = (split_on_k || !wseg) ? d0 : d1;
    dB = (split_on_k || wseg) ? d1 : d0;
    ldA = (split_on_k || !wseg) ? ld0 : ld1;
    ldB = (split_on_k || wseg) ? ld1 : ld0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int inst = wave * 8 + i;
      int o0, o1;
      if constexpr (MAJ == KMAJOR) {
        const int r = inst * 8 + (lane >> 3);
        const int c = (lane & 7) ^ kswz(r);
        const int R = r0 + r;
        const int R1 = split_on_k ? R : R - split;
        o0 = (R * ld0 + c * 8) * 2;
        o1 = (R1 * ld1 + c * 8) * 2;
      } else {
        const int blk = inst >> 3;
        const int kk = (inst & 7) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ oswz(kk);
        const int col = r0 + blk * 64 + c * 8;
        const int col1 = split_on_k ? col : col - split;
        o0 = (kk * ld0 + col) * 2;
        o1 = (kk * ld1 + col1) * 2;
      }
      offA[i] = (split_on_k || !wseg) ? o0 : o1;
      offB[i] = (split_on_k || wseg) ? o1 : o0;
    }
  }

  // Loads of the stage tile at k0 into LDS bytes [lds, +32 KB).  valid = 0
  // makes them out of range: they return zeros without touching memory
  // (buffer bounds) and keep the count of loads in flight fixed.
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int k0, bool valid) const {
    const bool kseg = split_on_k && k0 >= split;
    const int krel = kseg ? k0 - split : k0;
    const int kld = kseg ? ldB : ldA;
    const int soff = valid ? ((MAJ == KMAJOR) ? krel * 2 : krel * kld * 2) : kOutOfRange;
    const i32x4 d = kseg ? dB : dA;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lds_dma16(d, lds + (wave * 8 + i) * 1024, kseg ? offB[i] : offA[i], soff);
  }
};

// The same DMA with per-lane offsets by load parity (eight-wave kernel, where
// registers are scarcer): within a wave the swizzle depends on the load only
// through its parity (k-contiguous) or not at all (outer-contiguous), so a
// lane needs two offsets per segment and the rest of each load's address is
// wave-uniform (soffset).
template <int MAJ, int ESZ = 2>
struct StageLoaderP {
  static_assert(ESZ == 2 || (ESZ == 1 && MAJ == KMAJOR), "8-bit operands are k-contiguous");
  int vA[2], vB[2];  // per-lane byte offsets in segment A / B, [load parity]
  i32x4 dA, dB;      // buffer resources of segments A and B
  int ldA, ldB;      // leading dimensions (the k stride of outer-contiguous tiles)
  int rowA, rowB;    // k-contiguous: the wave's first row inside segment A / B
  int split, split_on_k;

  // segment A: segment 0 of a k-split operand, else the wave's segment;
  // segment B: segment 1 of a k-split operand, else the wave's segment
  __device__ __forceinline__ void init(const Operand& op, int r0, int wave, int lane) {
    const int ld0 = __builtin_amdgcn_readfirstlane(op.ld0);
    const int ld1 = __builtin_amdgcn_readfirstlane(op.ld1);
    split = __builtin_amdgcn_readfirstlane(op.split);
    split_on_k = __builtin_amdgcn_readfirstlane(op.split_on_k);
    const int wseg = (!split_on_k && r0 + 64 * wave >= split) ? 1 : 0;
    const bool a1 = !split_on_k && wseg;
    const bool b1 = split_on_k || wseg;
    const i32x4 d0 = make_desc(op.p0, op.bytes0), d1 = make_desc(op.p1, op.bytes1);
    dA = a1 ? d1 : d0;
    dB = b1 ? d1 : d0;
    ldA = a1 ? ld1 : ld0;
    ldB = b1 ? ld1 : ld0;
    const int outer_shift = wseg ? split : 0;  // outer index origin of the wave's segment
    const int lr = lane >> 3;
    if constexpr (MAJ == KMAJOR) {
      // load i covers rows 64 * wave + 8 * i + lr
      rowA = rowB = r0 + 64 * wave - outer_shift;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int c = (lane & 7) ^ kswz(8 * par + lr);
        vA[par] = ESZ == 2 ? (lr * ldA + c * 8) * 2 : lr * ldA + c * 16;
        vB[par] = ESZ == 2 ? (lr * ldB + c * 8) * 2 : lr * ldB + c * 16;
      }
    } else {
      // load i covers k-rows 8 * i + lr of outer block `wave`
      rowA = rowB = 0;
      const int c = (lane & 7) ^ oswz(lr);
      const int col = r0 + 64 * wave + c * 8 - outer_shift;
      vA[0] = vA[1] = (lr * ldA + col) * 2;
      vB[0] = vB[1] = (lr * ldB + col) * 2;
    }
  }

  // as StageLoader::issue
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int k0, bool valid) const {
    const bool kseg = split_on_k && k0 >= split;
    const int krel = kseg ? k0 - split : k0;
    const int ld = kseg ? ldB : ldA;
    const int row = kseg ? rowB : rowA;
    const i32x4 d = kseg ? dB : dA;
    const int v0 = kseg ? vB[0] : vA[0], v1 = kseg ? vB[1] : vA[1];
    int soff = (MAJ == KMAJOR) ? (row * ld + krel) * ESZ : krel * ld * 2;
    int step = 8 * ld * ESZ;  // 8 rows (or 8 k-rows) further per load
    if (!valid) { soff = kOutOfRange; step = 0; }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lds_dma16(d, lds + (wave * 8 + i) * 1024, (i & 1) ? v1 : v0, soff + i * step);
  }
  // load i (0..7) of issue alone
  __device__ __forceinline__ void issue_one(uint32_t lds, int wave, int k0, bool valid, int i) const {
    const bool kseg = split_on_k && k0 >= split;
    const int krel = kseg ? k0 - split : k0;
    const int ld = kseg ? ldB : ldA;
    const int row = kseg ? rowB : rowA;
    const i32x4 d = kseg ? dB : dA;
    const int v0 = kseg ? vB[0] : vA[0], v1 = kseg ? vB[1] : vA[1];
    int soff = (MAJ == KMAJOR) ? (row * ld + krel) * ESZ : krel * ld * 2;
    int step = 8 * ld * ESZ;
    if (!valid) { soff = kOutOfRange; step = 0; }
    lds_dma16(d, lds + (wave * 8 + i) * 1024, (i & 1) ? v1 : v0, soff + i * step);
  }
};

// The same stage tile loaded through registers instead (global -> VGPR ->
// ds_write_b128; used by the four-wave kernel): load i of wave w carries the
// same 1 KB as DMA load 8w + i and is written to the same LDS bytes.  The lane's offset depends only on
// the lane (and, for k-contiguous tiles, on the parity of i); the rest is
// wave-uniform and goes in soffset, which the buffer range check includes
// like the lane offset (zeros past the end, out-of-range loads included).
template <int MAJ>
struct RegLoader {
  int vA[2], vB[2];       // per-lane byte offsets in segment A / B, [load parity]
  const u16* pA;
  const u16* pB;
  int nA, nB, ldA, ldB;   // segment bytes and leading dimensions
  int rowA, rowB;         // k-contiguous: the wave's first row inside its segment
  int split, split_on_k;

  __device__ __forceinline__ void init(const Operand& op, int r0, int wave, int lane) {
    const int ld0 = __builtin_amdgcn_readfirstlane(op.ld0);
    const int ld1 = __builtin_amdgcn_readfirstlane(op.ld1);
    split = __builtin_amdgcn_readfirstlane(op.split);
    split_on_k = __builtin_amdgcn_readfirstlane(op.split_on_k);
    const int wseg = (!split_on_k && r0 + 64 * wave >= split) ? 1 : 0;
    const bool a1 = !split_on_k && wseg;       // segment of A
    const bool b1 = split_on_k || wseg;        // segment of B
    pA = a1 ? op.p1 : op.p0;
    pB = b1 ? op.p1 : op.p0;
    nA = __builtin_amdgcn_readfirstlane((int)(a1 ? op.bytes1 : op.bytes0));
    nB = __builtin_amdgcn_readfirstlane((int)(b1 ? op.bytes1 : op.bytes0));
    ldA = a1 ? ld1 : ld0;
    ldB = b1 ? ld1 : ld0;
    const int outer_shift = wseg ? split : 0;  // outer index origin of the wave's segment
    const int lr = lane >> 3;
    if constexpr (MAJ == KMAJOR) {
      rowA = r0 + 64 * wave - outer_shift;
      rowB = r0 + 64 * wave - outer_shift;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int c = (lane & 7) ^ ((par * 4 + (lr >> 1)) & 7);
        vA[par] = (lr * ldA + c * 8) * 2;
        vB[par] = (lr * ldB + c * 8) * 2;
      }
    } else {
      rowA = rowB = 0;
      const int c = (lane & 7) ^ oswz(lr);
      const int col = r0 + 64 * wave + c * 8 - outer_shift;
      vA[0] = vA[1] = (lr * ldA + col) * 2;
      vB[0] = vB[1] = (lr * ldB + col) * 2;
    }
  }

  __device__ __forceinline__ void load(int k0, bool valid, v4u* out) const {
    const bool kseg = split_on_k && k0 >= split;
    const int krel = kseg ? k0 - split : k0;
    const int ld = kseg ? ldB : ldA;
    const int row = kseg ? rowB : rowA;
    // wave-uniform by construction; keep descriptor and offsets scalar (a
    // value the compiler thinks divergent would get a per-lane loop)
    const uint64_t pa = reinterpret_cast<uint64_t>(kseg ? pB : pA);
    const uint32_t plo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pa));
    const uint32_t phi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pa >> 32));
    const u16* p = reinterpret_cast<const u16*>((static_cast<uint64_t>(phi) << 32) | plo);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(p), (short)0, __builtin_amdgcn_readfirstlane(kseg ? nB : nA), 0x00020000);
    const int v0 = kseg ? vB[0] : vA[0], v1 = kseg ? vB[1] : vA[1];
    int soff = (MAJ == KMAJOR) ? (row * ld + krel) * 2 : krel * ld * 2;
    int step = 16 * ld;  // 8 rows (or 8 k-rows) further per load
    if (!valid) { soff = kOutOfRange; step = 0; }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i & 1) ? v1 : v0,
                                                     __builtin_amdgcn_readfirstlane(soff + i * step), 0);
  }
};

// MFMA operand fragment for rows (or columns) [rb, rb + 32) and k-step ks
// (16 k) of a stage tile: lane l gets X[rb + l % 32][16 ks + 8 (l / 32) .. +7].
// For k-contiguous tiles koff is the lane's element offset of k-step ks in any
// 32-row block (rb a multiple of 32 leaves the swizzle unchanged), so a
// fragment's address is one register plus an immediate.
__device__ __forceinline__ int kfrag_offset(int ks, int lane) {
  const int r = lane & 31, c = ks * 2 + (lane >> 5);
  return r * BK + ((c ^ kswz(r)) << 3);
}

// The same fragment with the address computed in full (four-wave kernel).
template <int MAJ>
__device__ __forceinline__ bf16x8 frag4(const u16* tile, int rb, int ks, int lane) {
  if constexpr (MAJ == KMAJOR) {
    const int r = rb + (lane & 31), c = ks * 2 + (lane >> 5);
    return as_bf16x8(*reinterpret_cast<const uint4*>(tile + r * BK + ((c ^ kswz(r)) << 3)));
  } else {
    return frag_outer<BK>(tile, rb, ks, lane);
  }
}

template <int MAJ>
__device__ __forceinline__ bf16x8 frag(const u16* tile, int rb, int ks, int lane, int koff) {
  if constexpr (MAJ == KMAJOR) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(tile + rb * BK + koff));
  } else {
    static_assert(BK == 64, "outer-contiguous tiles are [64][64 k][64]");
    return frag_outer<BK>(tile, rb, ks, lane);
  }
}

// ---- epilogue
__device__ __forceinline__ void store16bf(u16* p, const float* v) {
  uint4 a, b;
  a.x = pack2bf(v[0], v[1]);   a.y = pack2bf(v[2], v[3]);
  a.z = pack2bf(v[4], v[5]);   a.w = pack2bf(v[6], v[7]);
  b.x = pack2bf(v[8], v[9]);   b.y = pack2bf(v[10], v[11]);
  b.z = pack2bf(v[12], v[13]); b.w = pack2bf(v[14], v[15]);
  reinterpret_cast<uint4*>(p)[0] = a;
  reinterpret_cast<uint4*>(p)[1] = b;
}

__device__ __forceinline__ void store16h(u16* p, const float* v) {
  uint4 a, b;
  a.x = pack2h(v[0], v[1]);   a.y = pack2h(v[2], v[3]);
  a.z = pack2h(v[4], v[5]);   a.w = pack2h(v[6], v[7]);
  b.x = pack2h(v[8], v[9]);   b.y = pack2h(v[10], v[11]);
  b.z = pack2h(v[12], v[13]); b.w = pack2h(v[14], v[15]);
  reinterpret_cast<uint4*>(p)[0] = a;
  reinterpret_cast<uint4*>(p)[1] = b;
}

__device__ __forceinline__ void load16bf(const u16* p, float* v) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) { v[2 * i] = lo_bf(w[i]); v[2 * i + 1] = hi_bf(w[i]); }
}

// Apply the epilogue to v[0..15] = C[r][c .. c+15].  `region` is the
// wave-uniform side of the split the 32 x 32 block lies on (split points are
// multiples of 64, blocks start at multiples of 32).
// SwiGLU pair (EPI_QKV_SWIGLU, FC1 side): u1[0..15] and u3[0..15] are the
// same rows and columns of a W1 block and its W3 block, cc the FC1-side
// column of u1's first value.
__device__ __forceinline__ void epi_swiglu16(const Epilogue& e, int r, int cc, float* u1,
                                             float* u3) {
  const int j = cc >> 6, w = cc & 31;
  store16bf(e.o1 + r * e.ld1 + cc, u1);
  store16bf(e.o1 + r * e.ld1 + cc + 32, u3);
#pragma unroll
  for (int i = 0; i < 16; ++i) u1[i] = silu_f(u1[i]) * u3[i];
  store16bf(e.o2 + r * e.ld2 + 32 * j + w, u1);
}

// DROP: the residual epilogue may drop (bf16 products; FP8 layers take no
// dropout, and leaving the mask code out keeps the four-wave kernel's
// unrolled epilogue small enough to keep its accumulators in registers)
template <int MODE, bool DROP = true>
__device__ __forceinline__ void epi_row16(const Epilogue& e, int region, int r, int c, float* v) {
  if constexpr (MODE == EPI_QKV_GELU || MODE == EPI_QKV_SWIGLU) {
    const int gc = c + e.col_base;
    if (region == 0) {  // the q, k columns: bf16 and fp16 copies
      store16bf(e.o0 + r * e.ld0 + gc, v);
      store16h(e.o3 + r * e.ld3 + gc, v);
    } else if (region == 1 || MODE == EPI_QKV_SWIGLU) {  // SwiGLU's FC1 side: epi_swiglu16
      store16bf(e.o0 + r * e.ld0 + gc, v);
    } else {
      const int cc = gc - e.split;
      store16bf(e.o1 + r * e.ld1 + cc, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = gelu_f(v[i]);
      store16bf(e.o2 + r * e.ld1 + cc, v);
    }
  } else if constexpr (MODE == EPI_RESIDUAL) {
    if (DROP && e.drop.on) dropout16(e.drop, static_cast<uint32_t>(r * e.ld0 + c), v);
    float xr[16];
    load16bf(e.i0 + r * e.ld0 + c, xr);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] += xr[i];
    store16bf(e.o0 + r * e.ld0 + c, v);
  } else if constexpr (MODE == EPI_DGELU) {
    if (region == 0) {
      store16bf(e.o0 + r * e.ld0 + c, v);
    } else {
      const int cc = c - e.split;
      float u[16];
      load16bf(e.i0 + r * e.ld2 + cc, u);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] *= gelu_grad_f(u[i]);
      store16bf(e.o1 + r * e.ld1 + e.col_off1 + cc, v);
    }
  } else if constexpr (MODE == EPI_DSWIGLU) {
    if (region == 0) {
      store16bf(e.o0 + r * e.ld0 + c, v);
    } else {
      const int cc = c - e.split;
      const int uc = 64 * (cc >> 5) + (cc & 31);
      float u1[16], u3[16];
      load16bf(e.i0 + r * e.ld2 + uc, u1);
      load16bf(e.i0 + r * e.ld2 + uc + 32, u3);
      float d1[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        d1[i] = v[i] * u3[i] * silu_grad_f(u1[i]);
        v[i] = v[i] * silu_f(u1[i]);
      }
      store16bf(e.o1 + r * e.ld1 + e.col_off1 + uc, d1);
      store16bf(e.o1 + r * e.ld1 + e.col_off1 + uc + 32, v);
    }
  } else if constexpr (MODE == EPI_STORE2_COLS) {
    if (region == 0) store16bf(e.o0 + r * e.ld0 + c, v);
    else store16bf(e.o1 + r * e.ld1 + (c - e.split), v);
  } else if constexpr (MODE == EPI_STORE2_ROWS) {
    if (region == 0) store16bf(e.o0 + r * e.ld0 + c, v);
    else store16bf(e.o1 + (r - e.split) * e.ld1 + c, v);
  } else {
    float4* o = reinterpret_cast<float4*>(e.of + r * e.ld0 + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <int MODE>
__device__ __forceinline__ int epi_region(const Epilogue& e, int r0, int cb) {
  if constexpr (MODE == EPI_QKV_GELU || MODE == EPI_QKV_SWIGLU) {
    const int g = cb + e.col_base;
    return g < e.lo_cols ? 0 : (g < e.split ? 1 : 2);
  } else if constexpr (MODE == EPI_DGELU || MODE == EPI_DSWIGLU || MODE == EPI_STORE2_COLS) {
    return cb < e.split ? 0 : 1;
  } else if constexpr (MODE == EPI_STORE2_ROWS) {
    return r0 < e.split ? 0 : 1;
  } else {
    return 0;
  }
}

// The fp32 partial sums of split tiles, stored and loaded at device (agent)
// scope: coherent across the XCDs, whose L2s are not, without writing back or
// invalidating a whole L2 as a fence would.  The cache policy is the one the
// compiler gives relaxed agent-scope atomics (sc1), here on 16-byte buffer
// accesses: a lane's 16 values of a 32 x 32 block sit as four float4 at
// [quad][lane], so one access of a quad covers 1 KB contiguous.  Offsets are
// bytes into the partial area (kGemmPartialBytes < 2^31).
constexpr int kCoherentPolicy = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* partials) {
  return __builtin_amdgcn_make_buffer_rsrc(partials, static_cast<short>(0),
                                           static_cast<int>(kGemmPartialBytes), 0x00020000);
}
__device__ __forceinline__ void store_part16(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                             const float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4u d = {__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                   __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, static_cast<int>(off + 1024 * q), 0,
                                           kCoherentPolicy);
  }
}
__device__ __forceinline__ void load_part16(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4u d =
        __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off + 1024 * q), 0, kCoherentPolicy);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q + e] = __uint_as_float(d[e]);
  }
}
// Byte offset of a lane's values of block `blk` (of 64 in a tile) in slot `slot`.
__device__ __forceinline__ uint32_t part_offset(int slot, int blk, int lane) {
  return static_cast<uint32_t>(slot) * (PARTIAL_FLOATS * 4) + blk * 4096 + lane * 16;
}

// Scheduling groups (instruction classes for __builtin_amdgcn_sched_group_barrier).
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// What one launch computes and how it is cut into work items.  An item is a
// k-range of one output tile; items are handed out in rounds, item i to
// workgroup i % G, so that the G items of a round run side by side at the
// same k positions (their operand panels meet in L2).
//   base items: tile t of problem p in `pieces[p]` k-pieces (pieces > 1
//     evens out the item lengths of two problems with different K), ordered
//     problem, then piece, then tile;
//   the first `full_items` base items (whole rounds) are items as they are;
//     each remaining base item is cut into `tail_split` k-pieces, so that the
//     last round still fills the CUs.
// A tile made of several items is summed by the last of them to finish.
struct SkPlan {
  GemmProblem p[2];
  int tiles_m[2], tiles_n[2], tiles[2];
  int iters[2];      // k-steps per tile
  int pieces[2];     // base k-pieces per tile
  int base0;         // base items of problem 0 (tiles[0] * pieces[0])
  int full_items;    // base items taken whole (whole rounds)
  int tail_split;    // k-pieces per remaining base item
  int nitems;
  int full_slots;    // partial slots of whole-round items (0 when none is split)
  float* partials;   // kGemmPartialSlots slots of PARTIAL_FLOATS
  int* counters;     // arrival count per global tile: zero on entry, left zero
  const float* amax_a;  // FP8: amax of the operands (device), else null
  const float* amax_b;
  const uint32_t* scale_a;  // MX: block-scale words [k-step][row] of A and B, else null
  const uint32_t* scale_b;
  int scale_lda, scale_ldb;  // words per k-step (>= rows)
  uint32_t scale_bytes_a, scale_bytes_b;
};

struct Item {
  int prob, tile, gtile, m0, n0, kb, len;
};

__device__ __forceinline__ Item decode_item(const SkPlan& pl, int i) {
  int b, tp = 0, ts = 1;
  if (i < pl.full_items) {
    b = i;
  } else {
    const int j = i - pl.full_items;
    ts = pl.tail_split;
    b = pl.full_items + j / ts;
    tp = j % ts;
  }
  Item it;
  it.prob = b < pl.base0 ? 0 : 1;
  const int bb = it.prob ? b - pl.base0 : b;
  const int T = pl.tiles[it.prob];
  const int q = bb / T, t = bb % T;
  const int iters = pl.iters[it.prob], pc = pl.pieces[it.prob];
  const int kq0 = q * iters / pc, kq1 = (q + 1) * iters / pc;
  const int ln = kq1 - kq0;
  it.kb = kq0 + tp * ln / ts;
  it.len = kq0 + (tp + 1) * ln / ts - it.kb;
  it.tile = t;
  it.gtile = it.prob ? pl.tiles[0] + t : t;
  // tile coordinates: groups of GM tile rows, column-major inside a group
  const int tm_count = pl.tiles_m[it.prob], tn_count = pl.tiles_n[it.prob];
  const int span = GM * tn_count;
  const int first_m = (t / span) * GM;
  const int gsz = min(tm_count - first_m, GM);
  it.m0 = (first_m + (t % span) % gsz) * TILE;
  it.n0 = ((t % span) / gsz) * TILE;
  return it;
}

// Items that make up tile t of problem p: for each base piece q, the base
// item itself (whole round) or its tail_split pieces.  f(item) is called in
// a fixed order.
template <typename F>
__device__ __forceinline__ void for_each_part(const SkPlan& pl, int p, int t, F&& f) {
  const int first = p ? pl.base0 : 0;
  for (int q = 0; q < pl.pieces[p]; ++q) {
    const int b = first + q * pl.tiles[p] + t;
    if (b < pl.full_items) {
      f(b);
    } else {
      const int i0 = pl.full_items + (b - pl.full_items) * pl.tail_split;
      for (int tp = 0; tp < pl.tail_split; ++tp) f(i0 + tp);
    }
  }
}

__device__ __forceinline__ int part_slot(const SkPlan& pl, int i) {
  return i < pl.full_items ? i : pl.full_slots + (i - pl.full_items);
}

// FMT 0: bf16 operands; FP8 operands with per-tensor (current) scales
// otherwise, FMT - 1 = fa + 2 fb with fa, fb the operands' formats
// (Fp8Format: 0 E4M3, 1 E5M2).  Block-scaled FP8 runs on the four-wave
// kernel below.
// H0: problem 0's operands are fp16 (v_mfma_f32_32x32x16_f16), problem 1's
// bf16; the same tiles, layouts and loads carry both.
template <int AMAJ, int BMAJ, int MODE, int FMT = 0, bool H0 = false>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_sk_kernel(SkPlan pl) {
  static_assert(!H0 || FMT == 0, "fp16 operands are 16-bit");
  constexpr bool F8 = FMT != 0;
  constexpr int FA = F8 ? (FMT - 1) & 1 : 0, FB = F8 ? (FMT - 1) >> 1 : 0;
  constexpr int ESZ = F8 ? 1 : 2;          // operand bytes per element
  constexpr int KSTEP = BK * 2 / ESZ;      // k-values per stage tile (128-byte rows)
  static_assert(!F8 || (AMAJ == KMAJOR && BMAJ == KMAJOR), "FP8 operands are k-contiguous");
  constexpr int RA = (AMAJ == KMAJOR) ? FM : 2 * FM;  // LDS read instructions per k-step
  constexpr int RB = (BMAJ == KMAJOR) ? FN : 2 * FN;
  // Two stages of 64 KB.  The epilogue's staging area (8 waves x 32 rows x
  // EPI_LD fp32) lies in stage 1, which is idle from an item's last k-step
  // until the next item's second stage tile goes out after the epilogue.
  __shared__ __attribute__((aligned(1024))) u16 ring[NSTAGE * STAGE];
  __shared__ int arrival;
  float* const epi_stage = reinterpret_cast<float*>(ring + STAGE);
  static_assert(WAVES * 32 * EPI_LD * 4 <= STAGE * 2, "epilogue staging fits in one stage");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const bool loader = wave < LOADERS;

  // Workgroups go round-robin over the 8 XCDs; virtual id v gives each XCD a
  // contiguous run of ranges.
  const int G = gridDim.x;
  int v;
  {
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int base = G / 8, rem = G % 8;
    v = xcd * base + min(xcd, rem) + loc;
  }
  if (v >= pl.nitems) return;
  StageLoaderP<AMAJ, ESZ> la;
  StageLoaderP<BMAJ, ESZ> lb;
  int item = v;
  Item s = decode_item(pl, item);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_address(ring));
  const __amdgpu_buffer_rsrc_t prs = partial_rsrc(pl.partials);

  auto setup = [&](const Item& sg) {
    const GemmProblem& P = pl.p[sg.prob];
    la.init(P.A, sg.m0, wave, lane);
    lb.init(P.B, sg.n0, wave, lane);
  };
  // stage tile j of an item (k-step kb + j) into ring slot `slot`, by the
  // loader waves; past the item's end the loads are out of range (zeros, no
  // memory traffic)
  auto issue_to = [&](const Item& sg, int slot, int j) {
    if (!loader) return;
    const bool valid = j < sg.len;
    const int k0 = (sg.kb + (valid ? j : 0)) * KSTEP;
    const uint32_t lds = ring_lds + slot * (STAGE * 2);
    la.issue(lds, wave, k0, valid);
    lb.issue(lds + TILE * BK * 2, wave, k0, valid);
  };

  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = kfrag_offset(ks, lane);
  f32x16 acc[FM][FN];
  bf16x8 fa[2][FM], fb[2][FN];
  auto rd = [&](const u16* st, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[slot][i] = frag<AMAJ>(st, wm * WM + i * 32, ks, lane, koff[ks]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[slot][j] = frag<BMAJ>(st + TILE * BK, wn * WN + j * 32, ks, lane, koff[ks]);
  };
  auto mma = [&](int slot, auto f16) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (decltype(f16)::value)
          acc[i][j] = mfma32x32x16_f16(fa[slot][i], fb[slot][j], acc[i][j]);
        else
          acc[i][j] = mfma32x32x16(fa[slot][i], fb[slot][j], acc[i][j]);
      }
  };
  // FP8: the 32 bytes of bf16 k-steps 2 half and 2 half + 1 (64 k-values).
  i32x8 ga[2][FM], gb[2][FN];
  auto rd8 = [&](const u16* st, int half, int slot) {
    const int k0 = koff[2 * half], k1 = koff[2 * half + 1];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const u16* t = st + (wm * WM + i * 32) * BK;
      ga[slot][i] = cat8(*reinterpret_cast<const uint4*>(t + k0),
                         *reinterpret_cast<const uint4*>(t + k1));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const u16* t = st + TILE * BK + (wn * WN + j * 32) * BK;
      gb[slot][j] = cat8(*reinterpret_cast<const uint4*>(t + k0),
                         *reinterpret_cast<const uint4*>(t + k1));
    }
  };
  auto mma8 = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma32x32x64_f8<FA, FB>(ga[slot][i], gb[slot][j], acc[i][j]);
  };
  auto pin8 = [&]() {
    constexpr int R = 2 * (FM + FN);
#pragma unroll
    for (int i = 0; i < FM * FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - FM * FN, 0);
  };
  // LDS reads of the next k-step spread between this k-step's MFMAs
  auto pin = [&]() {
    constexpr int R = RA + RB;
#pragma unroll
    for (int i = 0; i < (R < FM * FN ? R : FM * FN); ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    if constexpr (R < FM * FN) __builtin_amdgcn_sched_group_barrier(SG_MFMA, FM * FN - R, 0);
    if constexpr (R > FM * FN) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - FM * FN, 0);
  };

  setup(s);
  issue_to(s, 0, 0);
  issue_to(s, 1, 1);
  for (;;) {
    // ---- main loop over the item's 64-wide k-steps, two stages: step j
    // computes stage tile j (4 MFMA k-steps of 16) while tile j+1 streams
    // in, then waits for it, and after the barrier the loads of tile j+2 go
    // into the stage just read (out of range past the item's end, so the
    // loop has no branch and no MFMA under one).  Fragments of the next
    // 16-wide k-step are read under the MFMAs of the current one.  Two waves
    // share each SIMD, so one wave's MFMAs cover the other's waits.
    const int len = s.len;
    // Every memory operation of this wave done, the first stage tiles
    // included.  A clean slate also keeps the compiler's own wait counting
    // from carrying the epilogue's loads and stores into the loop.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if constexpr (F8) {
      // the same pipeline with two FP8 MFMA steps of 64 k per stage tile
      rd8(ring, 0, 0);
      for (int j = 0; j < len; ++j) {
        u16* cur = ring + (j & 1) * STAGE;
        rd8(cur, 1, 1);
        mma8(0);
        pin8();
        wait_vm_lds<0>();
        __syncthreads();
        issue_to(s, j & 1, j + 2);
        rd8(ring + ((j + 1) & 1) * STAGE, 0, 0);  // unused after the last step
        mma8(1);
        pin8();
      }
    } else {
      auto loop16 = [&](auto f16) {
        rd(ring, 0, 0);
        for (int j = 0; j < len; ++j) {
          u16* cur = ring + (j & 1) * STAGE;
          rd(cur, 1, 1);
          mma(0, f16);
          pin();
          rd(cur, 2, 0);
          mma(1, f16);
          pin();
          rd(cur, 3, 1);
          mma(0, f16);
          pin();
          wait_vm_lds<0>();  // tile j+1 landed (the loader waves' loads)
          __syncthreads();   // tile j+1 in LDS for every wave; tile j read by every wave
          issue_to(s, j & 1, j + 2);
          rd(ring + ((j + 1) & 1) * STAGE, 0, 0);  // unused after the last step
          mma(1, f16);
          pin();
        }
      };
      if constexpr (H0) {
        if (s.prob == 0) loop16(std::true_type{});
        else loop16(std::false_type{});
      } else {
        loop16(std::false_type{});
      }
    }

    // ---- the next item's first stage tile goes out before this one's
    // epilogue (into stage 0; stage 1 holds the epilogue's staging)
    const int next = item + G;
    const bool more = next < pl.nitems;
    wait_vm_lds<0>();  // this item's trailing (out-of-range) loads are done
    __syncthreads();   // and every wave is done reading the ring
    Item nx;
    if (more) {
      nx = decode_item(pl, next);
      setup(nx);
      issue_to(nx, 0, 0);
    }

    // ---- finish the tile, one 32 x 32 block of each wave at a time: the
    // block goes through the wave's LDS staging area, after which lane l
    // holds row l / 2, columns 16 (l % 2) .. +15 of it.
    //   phase 0 (tile made of several items): store this item's fp32
    //     partial sums, then count it in; the last item to arrive goes on to
    //     phase 1 with all the partials;
    //   phase 1: the epilogue, on the sum of the tile's partials (in a fixed
    //     order, so the result does not depend on the order of arrival).
    // Partial slot layout: block (wave, i, j) of 4 KB, [quad][lane][4] fp32.
    {
      const GemmProblem& P = pl.p[s.prob];
      const Epilogue& e = P.epi;
      const int lrow = lane & 31, lk = lane >> 5;
      const int er = lane >> 1, ec = (lane & 1) * 16;
      float* ep = epi_stage + wave * 32 * EPI_LD;
      int nparts = 0;
      for_each_part(pl, s.prob, s.tile, [&](int) { ++nparts; });
      int phase = nparts > 1 ? 0 : 1;
      bool summed = false;  // phase 1 on a sum of partials
      const int my_slot = part_slot(pl, item);
      float held[MODE == EPI_QKV_SWIGLU ? 16 : 1];
      float dq = 1.0f;  // FP8: 1 / (sA sB)
      if constexpr (F8)
        dq = inv_scale(*pl.amax_a, fp8_max(FA)) * inv_scale(*pl.amax_b, fp8_max(FB));
      for (;;) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 16; ++q)
              ep[((q >> 2) * 8 + lk * 4 + (q & 3)) * EPI_LD + lrow] = acc[i][j][q];
            __builtin_amdgcn_wave_barrier();
            float vals[16];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float4 x = *reinterpret_cast<const float4*>(ep + er * EPI_LD + ec + 4 * t);
              vals[4 * t] = x.x; vals[4 * t + 1] = x.y; vals[4 * t + 2] = x.z; vals[4 * t + 3] = x.w;
            }
            __builtin_amdgcn_wave_barrier();
            // this lane's 16 values of the block (see store_part16)
            const int blk = (wave * FM + i) * FN + j;
            if (phase == 0) {
              store_part16(prs, part_offset(my_slot, blk, lane), vals);
            } else {
              if (summed) {
                // every piece's partial in the tile's fixed order; this
                // piece's own values are still at hand (the bits it stored)
                float own[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) own[t] = vals[t];
                bool first = true;
                for_each_part(pl, s.prob, s.tile, [&](int part) {
                  float x[16];
                  if (part == item) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) x[t] = own[t];
                  } else {
                    load_part16(prs, part_offset(part_slot(pl, part), blk, lane), x);
                  }
#pragma unroll
                  for (int t = 0; t < 16; ++t) vals[t] = first ? x[t] : vals[t] + x[t];
                  first = false;
                });
              }
              if constexpr (F8) {
#pragma unroll
                for (int t = 0; t < 16; ++t) vals[t] *= dq;
              }
              const int r0 = s.m0 + wm * WM + i * 32, cb = s.n0 + wn * WN + j * 32;
              const int region = __builtin_amdgcn_readfirstlane(epi_region<MODE>(e, r0, cb));
              const int r = r0 + er;
              if constexpr (MODE == EPI_QKV_SWIGLU) {
                // FC1 side: the wave's two blocks are W1 and W3 of the same
                // columns; block 0's values wait in `held` for block 1
                static_assert(FN == 2 && WN == 64, "a wave holds one W1 | W3 pair");
                if (region == 2) {
                  if (j == 0) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) held[t] = vals[t];
                  } else if (cb - 32 < P.N && r < P.M) {
                    epi_swiglu16(e, r, cb - 32 + e.col_base - e.split + ec, held, vals);
                  }
                } else if (cb < P.N && r < P.M) {
                  epi_row16<MODE, FMT == 0>(e, region, r, cb + ec, vals);
                }
              } else {
                if (cb < P.N && r < P.M) epi_row16<MODE, FMT == 0>(e, region, r, cb + ec, vals);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (phase == 1) break;
        // The partial is written at device scope (past the XCD's own L2);
        // every store of it has completed before the item counts itself in.
        wait_vm_lds<0>();
        __syncthreads();
        if (tid == 0) arrival = atomicAdd(pl.counters + s.gtile, 1);
        __syncthreads();
        const int arrived = __builtin_amdgcn_readfirstlane(arrival);
        if (arrived != nparts - 1) break;  // another item finishes this tile
        // last to arrive: the other partials are complete at device scope and
        // are read at device scope
        if (tid == 0) pl.counters[s.gtile] = 0;  // clean for the next launch
        phase = 1;
        summed = true;
      }
    }
    if (!more) break;
    __syncthreads();  // every wave done with the staging area in stage 1
    issue_to(nx, 1, 1);
    s = nx;
    item = next;
  }
}

// The four-wave kernel (one wave per SIMD, 128 x 128 outputs per wave, the
// accumulators in AGPRs), kept for the two products whose operands are both
// k-contiguous (the dgrad products): there A goes through registers (loaded
// at the start of a k-step, written at its end) and B by DMA, which splits
// the operand stream over both paths, and that measures faster than the
// eight-wave kernel's DMA-only stream.  Same items, epilogue and partials as
// the eight-wave kernel.
// MX: every product on block-scaled FP8 operands (FMT - 1 = fa + 2 fb).  The
// scaled MFMA needs about 20 registers more than the plain one, which the
// eight-wave kernel does not have; here the accumulators sit in AGPRs and the
// fragments of both halves of a stage tile fit in VGPRs.  Both operands go by
// DMA (32 KB each per 128-wide k-step), the tile's scale words (1 KB per
// operand) beside them into a small LDS ring.
template <int AMAJ, int BMAJ, int MODE, int FMT = 0, bool MX = false>
__global__ __launch_bounds__(256, 1) void gemm_kernel4(SkPlan pl) {
  constexpr bool F8 = FMT != 0;
  static_assert(!MX || F8, "block scales come with FP8 operands");
  static_assert(!F8 || (AMAJ == KMAJOR && BMAJ == KMAJOR), "FP8 operands are k-contiguous");
  constexpr int FA = F8 ? (FMT - 1) & 1 : 0, FB = F8 ? (FMT - 1) >> 1 : 0;
  constexpr int KSTEP = F8 ? 2 * BK : BK;  // k-values per stage tile (128-byte rows)
  constexpr int WM = 128, WN = 128, FM = 4, FN = 4;
  constexpr int RA = (AMAJ == KMAJOR) ? FM : 2 * FM;  // LDS read instructions per k-step
  constexpr int RB = (BMAJ == KMAJOR) ? FN : 2 * FN;
  __shared__ __attribute__((aligned(1024))) u16 ring[NSTAGE * STAGE];
  __shared__ __attribute__((aligned(16))) float epi_stage[4 * 32 * EPI_LD];
  // MX: per stage the scale words of the A tile's 256 rows, then the B tile's
  __shared__ __attribute__((aligned(1024))) uint32_t sring[MX ? NSTAGE * 2 * TILE : 1];
  __shared__ int arrival;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Workgroups go round-robin over the 8 XCDs; virtual id v gives each XCD a
  // contiguous run of ranges.
  const int G = gridDim.x;
  int v;
  {
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int base = G / 8, rem = G % 8;
    v = xcd * base + min(xcd, rem) + loc;
  }
  if (v >= pl.nitems) return;
  // Both operands k-contiguous (the two dgrad products): A goes through
  // registers and B by LDS DMA, which splits the operand stream over both
  // paths; otherwise both go by DMA (measured per product: see the notes on
  // the main loop).
  constexpr bool AREG = (AMAJ == KMAJOR && BMAJ == KMAJOR) && !F8;
  std::conditional_t<F8, StageLoaderP<KMAJOR, 1>,
                     std::conditional_t<AREG, RegLoader<AMAJ>, StageLoader<AMAJ>>> la;
  std::conditional_t<F8, StageLoaderP<KMAJOR, 1>, StageLoader<BMAJ>> lb;
  int item = v;
  Item s = decode_item(pl, item);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_address(ring));
  const uint32_t sring_lds = __builtin_amdgcn_readfirstlane(lds_address(sring));
  const __amdgpu_buffer_rsrc_t prs = partial_rsrc(pl.partials);
  const int sop = __builtin_amdgcn_readfirstlane(wave) & 1;  // MX: scale words staged by this wave
  const i32x4 sdesc = sop ? make_desc(reinterpret_cast<const u16*>(pl.scale_b), pl.scale_bytes_b)
                          : make_desc(reinterpret_cast<const u16*>(pl.scale_a), pl.scale_bytes_a);
  const int sld = sop ? pl.scale_ldb : pl.scale_lda;

  auto setup = [&](const Item& sg) {
    const GemmProblem& P = pl.p[sg.prob];
    la.init(P.A, sg.m0, wave, lane);
    lb.init(P.B, sg.n0, wave, lane);
  };
  // stage tile j (k-step kb + j of the segment) into ring slot j % 4
  // stage tile j of a segment (k-step kb + j) into ring slot st; past the
  // segment's end the loads are out of range (zeros, no memory traffic)
  auto issue_to = [&](const Item& sg, int slot, int j) {
    const bool valid = j < sg.len;
    const int k0 = (sg.kb + (valid ? j : 0)) * KSTEP;
    const uint32_t lds = ring_lds + slot * (STAGE * 2);
    if constexpr (!AREG) la.issue(lds, wave, k0, valid);
    lb.issue(lds + TILE * BK * 2, wave, k0, valid);
    if constexpr (MX) {
      // scale words of the tile's 256 rows at this k-step: 1 KB per operand,
      // one load per wave, of operand sop (A: 0, B: 1); waves 2 and 3 repeat
      // waves 0 and 1 (the same bytes to the same place), which keeps the
      // loop free of branches.  Rows past the array read as zero (their
      // operand rows are zero too).
      const int ks = sg.kb + (valid ? j : 0);
      const int row0 = sop ? sg.n0 : sg.m0;
      lds_dma16(sdesc, sring_lds + (slot * 2 + sop) * (TILE * 4), lane * 16,
                valid ? (ks * sld + row0) * 4 : kOutOfRange);
    }
  };
  // A through registers (AREG): load stage tile j of A, then write it to LDS
  v4u stg[AREG ? 8 : 1];
  auto gload_a = [&](const Item& sg, int j) {
    if constexpr (AREG) {
      const bool valid = j < sg.len;
      const int k0 = (sg.kb + (valid ? j : 0)) * BK;
      la.load(k0, valid, stg);
    }
  };
  auto commit_a = [&](int slot) {
    if constexpr (AREG) {
      u16* st = ring + slot * STAGE + wave * 4096 + lane * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<v4u*>(st + i * 512) = stg[i];
    }
  };
  auto prologue = [&](const Item& sg) {
    setup(sg);
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j) issue_to(sg, j, j);
    gload_a(sg, 0);
    commit_a(0);
  };

  f32x16 acc[FM][FN];
  bf16x8 fa[2][FM], fb[2][FN];
  auto rd = [&](const u16* st, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[slot][i] = frag4<AMAJ>(st, wm * WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[slot][j] = frag4<BMAJ>(st + TILE * BK, wn * WN + j * 32, ks, lane);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[slot][i], fb[slot][j], acc[i][j]);
  };
  // LDS reads of the next k-step spread between this k-step's MFMAs
  auto pin = [&]() {
    constexpr int R = RA + RB;
#pragma unroll
    for (int i = 0; i < (R < FM * FN ? R : FM * FN); ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    if constexpr (R < FM * FN) __builtin_amdgcn_sched_group_barrier(SG_MFMA, FM * FN - R, 0);
    if constexpr (R > FM * FN) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - FM * FN, 0);
  };
  // FP8: the 32 bytes of one 64-wide half of a stage tile per fragment (bf16
  // k-steps 2 half and 2 half + 1 of the same rows).  MX: lane half h' holds
  // k [64 half + 16 h', +16) and [64 half + 32 + 16 h', +16), so the matrix
  // cores' block b of this half is the tile's 32-wide block 2 half + b, whose
  // scale they take from lane half b.  In the scale layout (mx_scale_byte)
  // the lane finds the codes of its four fragments' rows for both halves in
  // 8 bytes, word 0 for half 0 and word 1 for half 1, byte i for fragment i:
  // the operands of the MFMA's immediate byte selects, one word per half
  // and operand, read with that half's fragments.
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = kfrag_offset(ks, lane);
  i32x8 ga[2][F8 ? FM : 1], gb[2][F8 ? FN : 1];
  uint32_t sa8[2], sb8[2];
  const int srec = 4 * (lane & 31) + 2 * (lane >> 5);  // the lane's 8 bytes, in words
  auto rd8 = [&](const u16* st, int half, int slot) {
    if constexpr (F8) {
      const int k0 = koff[2 * half], k1 = koff[2 * half + 1];
      if constexpr (MX) {
        const uint32_t* sw = sring + ((st - ring) / STAGE) * (2 * TILE) + srec + half;
        sa8[slot] = sw[wm * WM];
        sb8[slot] = sw[TILE + wn * WN];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const u16* t = st + (wm * WM + i * 32) * BK;
        ga[slot][i] = cat8(*reinterpret_cast<const uint4*>(t + k0),
                           *reinterpret_cast<const uint4*>(t + k1));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const u16* t = st + TILE * BK + (wn * WN + j * 32) * BK;
        gb[slot][j] = cat8(*reinterpret_cast<const uint4*>(t + k0),
                           *reinterpret_cast<const uint4*>(t + k1));
      }
    }
  };
  auto mma8 = [&](int slot) {
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mx_step4<FA, FB>(i, j, ga[slot][i], gb[slot][j], acc[i][j], sa8[slot],
                                       sb8[slot]);
    } else if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32x32x64_f8<FA, FB>(ga[slot][i], gb[slot][j], acc[i][j]);
    }
  };
  // the next half's fragment reads (half 0: and the scale reads) between
  // this half's MFMAs
  auto pin8 = [&](auto next_half) {
    constexpr int R = 2 * (FM + FN) + (MX ? 2 : 0);
#pragma unroll
    for (int i = 0; i < FM * FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    if constexpr (R > FM * FN) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - FM * FN, 0);
  };

  // FP8, after a k-step's barrier: the half-step's sixteen MFMAs (slot 1),
  // each followed by one DMA load of the stage tile after next and one
  // fragment read of the next half (slot 0).  A DMA issue can wait for room
  // in the memory pipeline's queue; placed after an MFMA it waits while that
  // MFMA runs instead of holding up the MFMAs behind it.  Two empty asm
  // statements (they emit nothing) hold the order, being ordered with the
  // DMA as asm with side effects: one takes the MFMA's result as an input,
  // so the MFMA cannot sink below the DMA after it, the other claims to
  // rewrite an operand of the next MFMA, so that one cannot rise above it.
  auto half_dma8 = [&](const Item& sg, int slot, int j, const u16* st) {
    if constexpr (F8) {
      static_assert(FM * FN == 16 && 2 * (FM + FN) == 16, "one load and one read per MFMA");
      const bool valid = j < sg.len;
      const int k0 = (sg.kb + (valid ? j : 0)) * KSTEP;
      const uint32_t lds = ring_lds + slot * (STAGE * 2);
      const int k0f = koff[0], k1f = koff[1];
      uint4 x0;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int i = t / FN, jj = t % FN;
        if (t > 0) asm volatile("" : "+v"(gb[1][jj]));
        if constexpr (MX)
          acc[i][jj] = mx_step4<FA, FB>(i, jj, ga[1][i], gb[1][jj], acc[i][jj], sa8[1], sb8[1]);
        else
          acc[i][jj] = mfma32x32x64_f8<FA, FB>(ga[1][i], gb[1][jj], acc[i][jj]);
        asm volatile("" ::"a"(acc[i][jj]));
        if (t < 8) la.issue_one(lds, wave, k0, valid, t);
        else lb.issue_one(lds + TILE * BK * 2, wave, k0, valid, t - 8);
        const int f = (t & 7) >> 1;
        const u16* base = t < 8 ? st + (wm * WM + f * 32) * BK
                                : st + TILE * BK + (wn * WN + f * 32) * BK;
        const uint4 x = *reinterpret_cast<const uint4*>(base + ((t & 1) ? k1f : k0f));
        if ((t & 1) == 0) x0 = x;
        else if (t < 8) ga[0][f] = cat8(x0, x);
        else gb[0][f] = cat8(x0, x);
      }
      if constexpr (MX) {
        const int ks = sg.kb + (valid ? j : 0);
        const int row0 = sop ? sg.n0 : sg.m0;
        lds_dma16(sdesc, sring_lds + (slot * 2 + sop) * (TILE * 4), lane * 16,
                  valid ? (ks * sld + row0) * 4 : kOutOfRange);
        const uint32_t* sw = sring + ((st - ring) / STAGE) * (2 * TILE) + srec;
        sa8[0] = sw[wm * WM];
        sb8[0] = sw[TILE + wn * WN];
      }
    }
  };

  prologue(s);
  for (;;) {
    // ---- main loop over the segment's 64-wide k-steps, two stages: step j
    // computes stage tile j (4 MFMA k-steps of 16) while tile j+1 streams
    // in, then waits for it, and after the barrier the loads of tile j+2 go
    // into the stage just read (out of range past the segment's end, so the
    // loop has no branch and no MFMA under one).  Fragments of the next
    // 16-wide k-step are read under the MFMAs of the current one.
    const int len = s.len;
    // Every memory operation of this wave done, the first stage tiles
    // included (they went out before the previous tile's epilogue).  A clean
    // slate here also keeps the compiler's own wait counting from carrying
    // the epilogue's loads and stores into the loop.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if constexpr (F8) {
      // two FP8 MFMA half-steps of 64 k per 128-wide stage tile
      rd8(ring, 0, 0);
      for (int j = 0; j < len; ++j) {
        u16* cur = ring + (j & 1) * STAGE;
        rd8(cur, 1, 1);
        mma8(0);
        pin8(std::integral_constant<int, 1>{});
        wait_vm_lds<0>();  // tile j+1 landed (operands and scale words)
        __syncthreads();   // tile j+1 in LDS for every wave; tile j read by every wave
        // tile j+2's loads; the reads are unused after the last step
        half_dma8(s, j & 1, j + 2, ring + ((j + 1) & 1) * STAGE);
      }
    } else if constexpr (AREG) {
      rd(ring, 0, 0);
      // A's tile j+1 is loaded into registers at the start of step j (its
      // loads spread between the first k-step's MFMAs) and written to the
      // free stage at the end; B's tile j+2 goes by DMA after the barrier.
      for (int j = 0; j < len; ++j) {
        u16* cur = ring + (j & 1) * STAGE;
        gload_a(s, j + 1);
        rd(cur, 1, 1);
        mma(0);
#pragma unroll
        for (int i = 0; i < FM * FN; ++i) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
        }
        rd(cur, 2, 0);
        mma(1);
        pin();
        rd(cur, 3, 1);
        mma(0);
        pin();
        commit_a((j + 1) & 1);
        wait_vm_lds<0>();  // B's tile j+1 landed, A's written
        __syncthreads();   // tile j+1 in LDS for every wave; tile j read by every wave
        issue_to(s, j & 1, j + 2);
        rd(ring + ((j + 1) & 1) * STAGE, 0, 0);  // unused after the last step
        mma(1);
        pin();
      }
    } else {
      rd(ring, 0, 0);
      for (int j = 0; j < len; ++j) {
        u16* cur = ring + (j & 1) * STAGE;
        rd(cur, 1, 1);
        mma(0);
        pin();
        rd(cur, 2, 0);
        mma(1);
        pin();
        rd(cur, 3, 1);
        mma(0);
        pin();
        wait_vm_lds<0>();  // tile j+1 landed
        __syncthreads();   // tile j+1 in LDS for every wave; tile j read by every wave
        issue_to(s, j & 1, j + 2);
        rd(ring + ((j + 1) & 1) * STAGE, 0, 0);  // unused after the last step
        mma(1);
        pin();
      }
    }

    // ---- the next item's first stage tiles go out before this one's epilogue
    const int next = item + G;
    const bool more = next < pl.nitems;
    Item nx;
    if (more) {
      wait_vm_lds<0>();  // this item's trailing (out-of-range) loads are done
      __syncthreads();   // and every wave is done reading the ring
      nx = decode_item(pl, next);
      // with A through registers the staging registers would stay live
      // across the epilogue; that prologue runs after it instead
      if constexpr (!AREG) prologue(nx);
    }

    // ---- finish the tile, one 32 x 32 block of each wave at a time: the
    // block goes through the wave's LDS staging area, after which lane l
    // holds row l / 2, columns 16 (l % 2) .. +15 of it.
    //   phase 0 (tile made of several items): store this item's fp32
    //     partial sums, then count it in; the last item to arrive goes on to
    //     phase 1 with all the partials;
    //   phase 1: the epilogue, on the sum of the tile's partials (in a fixed
    //     order, so the result does not depend on the order of arrival).
    // Partial slot layout: block (wave, i, j) of 4 KB, [quad][lane][4] fp32.
    {
      const GemmProblem& P = pl.p[s.prob];
      const Epilogue& e = P.epi;
      const int lrow = lane & 31, lk = lane >> 5;
      const int er = lane >> 1, ec = (lane & 1) * 16;
      float* ep = epi_stage + wave * 32 * EPI_LD;
      int nparts = 0;
      for_each_part(pl, s.prob, s.tile, [&](int) { ++nparts; });
      int phase = nparts > 1 ? 0 : 1;
      bool summed = false;  // phase 1 on a sum of partials
      const int my_slot = part_slot(pl, item);
      float dq = 1.0f;  // FP8 with per-tensor scales: 1 / (sA sB)
      if constexpr (F8 && !MX)
        dq = inv_scale(*pl.amax_a, fp8_max(FA)) * inv_scale(*pl.amax_b, fp8_max(FB));
      for (;;) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 16; ++q)
              ep[((q >> 2) * 8 + lk * 4 + (q & 3)) * EPI_LD + lrow] = acc[i][j][q];
            __builtin_amdgcn_wave_barrier();
            float vals[16];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float4 x = *reinterpret_cast<const float4*>(ep + er * EPI_LD + ec + 4 * t);
              vals[4 * t] = x.x; vals[4 * t + 1] = x.y; vals[4 * t + 2] = x.z; vals[4 * t + 3] = x.w;
            }
            __builtin_amdgcn_wave_barrier();
            // this lane's 16 values of the block (see store_part16)
            const int blk = (wave * FM + i) * FN + j;
            if (phase == 0) {
              store_part16(prs, part_offset(my_slot, blk, lane), vals);
            } else {
              if (summed) {
                // every piece's partial in the tile's fixed order; this
                // piece's own values are still at hand (the bits it stored)
                float own[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) own[t] = vals[t];
                bool first = true;
                for_each_part(pl, s.prob, s.tile, [&](int part) {
                  float x[16];
                  if (part == item) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) x[t] = own[t];
                  } else {
                    load_part16(prs, part_offset(part_slot(pl, part), blk, lane), x);
                  }
#pragma unroll
                  for (int t = 0; t < 16; ++t) vals[t] = first ? x[t] : vals[t] + x[t];
                  first = false;
                });
              }
              if constexpr (F8 && !MX) {
#pragma unroll
                for (int t = 0; t < 16; ++t) vals[t] *= dq;
              }
              const int r0 = s.m0 + wm * WM + i * 32, cb = s.n0 + wn * WN + j * 32;
              const int region = __builtin_amdgcn_readfirstlane(epi_region<MODE>(e, r0, cb));
              const int r = r0 + er;
              if (cb < P.N && r < P.M) epi_row16<MODE, FMT == 0>(e, region, r, cb + ec, vals);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (phase == 1) break;
        // The partial is written at device scope (past the XCD's own L2);
        // every store of it has completed before the item counts itself in.
        wait_vm_lds<0>();
        __syncthreads();
        if (tid == 0) arrival = atomicAdd(pl.counters + s.gtile, 1);
        __syncthreads();
        const int arrived = __builtin_amdgcn_readfirstlane(arrival);
        if (arrived != nparts - 1) break;  // another item finishes this tile
        // last to arrive: the other partials are complete at device scope and
        // are read at device scope
        if (tid == 0) pl.counters[s.gtile] = 0;  // clean for the next launch
        phase = 1;
        summed = true;
      }
    }
    if (!more) break;
    if constexpr (AREG) prologue(nx);
    s = nx;
    item = next;
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// Compute units of the current device, cached per device.  The cache is the
// library's one piece of mutable global state besides the per-device address
// of its static scratch array: each slot only ever goes from 0 to the
// device's count, with relaxed atomics, so concurrent first calls are benign.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && n > 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int tiles_of(int M, int N) { return ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE); }

bool operand_ok(const Operand& op) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  // one-segment operands put the split out of reach (INT_MAX)
  return al(op.p0) && al(op.p1) && op.ld0 % 8 == 0 && op.ld1 % 8 == 0 && op.ld0 > 0 &&
         op.ld1 > 0 && op.split >= 0 && (op.split % 64 == 0 || op.split >= (1 << 30));
}

// FP8 products run on the four-wave kernel, except the weight gradients
// with current scales (E4M3 x E5M2): their k-extent is the token count, a
// short main loop per tile, and there the eight-wave kernel, whose epilogue
// is spread over twice the waves, measured faster.
template <int MODE, int FMT, bool MX = false>
hipError_t launch_plan_fp8(const SkPlan& pl, int grid, hipStream_t s) {
  if constexpr (!MX && FMT - 1 == FP8_E4M3 + 2 * FP8_E5M2)
    hipLaunchKernelGGL((gemm_sk_kernel<KMAJOR, KMAJOR, MODE, FMT>), dim3(grid), dim3(64 * WAVES),
                       0, s, pl);
  else
    hipLaunchKernelGGL((gemm_kernel4<KMAJOR, KMAJOR, MODE, FMT, MX>), dim3(grid), dim3(256), 0, s,
                       pl);
  return hipGetLastError();
}

template <int AMAJ, int BMAJ, int MODE, bool H0 = false>
hipError_t launch_plan(const SkPlan& pl, int grid, hipStream_t s) {
  static_assert(!H0 || !(AMAJ == KMAJOR && BMAJ == KMAJOR), "fp16 problems run on eight waves");
  if constexpr (AMAJ == KMAJOR && BMAJ == KMAJOR)
    hipLaunchKernelGGL((gemm_kernel4<AMAJ, BMAJ, MODE>), dim3(grid), dim3(256), 0, s, pl);
  else
    hipLaunchKernelGGL((gemm_sk_kernel<AMAJ, BMAJ, MODE, 0, H0>), dim3(grid),
                       dim3(64 * WAVES), 0, s, pl);
  return hipGetLastError();
}

// Cut the work of one launch into items (see SkPlan).  `tail_split` > 0
// forces the k-pieces of the last round's base items (tests and tuning);
// 0 picks enough pieces to fill the CUs, at least 16 k-steps each.  kstep:
// k-values per stage tile (64 bf16, 128 FP8).
hipError_t build_plan(const GemmProblem* probs, int nprob, Major a_major, Major b_major,
                      const GemmScratch& ws, int tail_split, SkPlan* out, int* grid_out,
                      int kstep = BK) {
  if (nprob < 1 || nprob > 2) return hipErrorInvalidValue;
  SkPlan pl;
  for (int i = 0; i < 2; ++i) {
    const GemmProblem& p = probs[i < nprob ? i : 0];
    // the epilogue writes 16 consecutive columns at a time
    if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.N % 16 != 0) return hipErrorInvalidValue;
    // k-contiguous operands are read in whole k-steps
    if ((a_major == KMAJOR || b_major == KMAJOR) && p.K % kstep != 0) return hipErrorInvalidValue;
    if (!operand_ok(p.A) || !operand_ok(p.B)) return hipErrorInvalidValue;
    pl.p[i] = p;
    pl.tiles_m[i] = (p.M + TILE - 1) / TILE;
    pl.tiles_n[i] = (p.N + TILE - 1) / TILE;
    pl.iters[i] = (p.K + kstep - 1) / kstep;
  }
  const long t0 = static_cast<long>(pl.tiles_m[0]) * pl.tiles_n[0];
  const long t1 = nprob > 1 ? static_cast<long>(pl.tiles_m[1]) * pl.tiles_n[1] : 0;
  if (t0 + t1 > ws.max_tiles || t0 + t1 >= (1L << 24)) return hipErrorInvalidValue;
  pl.tiles[0] = static_cast<int>(t0);
  pl.tiles[1] = static_cast<int>(t1);
  pl.partials = ws.partials;
  pl.counters = ws.counters;
  pl.amax_a = pl.amax_b = nullptr;
  pl.scale_a = pl.scale_b = nullptr;
  pl.scale_lda = pl.scale_ldb = 0;
  pl.scale_bytes_a = pl.scale_bytes_b = 0;

  int G = device_cus();
  if (G <= 0) return hipErrorInvalidDevice;
  if (G > kGemmMaxWorkgroups) G = kGemmMaxWorkgroups;
  for (int attempt = 0; attempt < 2; ++attempt) {
    // equal item lengths for two problems whose K differ by a whole factor
    pl.pieces[0] = pl.pieces[1] = 1;
    if (attempt == 0 && t1 > 0) {
      if (pl.iters[0] > pl.iters[1] && pl.iters[0] % pl.iters[1] == 0)
        pl.pieces[0] = pl.iters[0] / pl.iters[1];
      else if (pl.iters[1] > pl.iters[0] && pl.iters[1] % pl.iters[0] == 0)
        pl.pieces[1] = pl.iters[1] / pl.iters[0];
    }
    const long base0 = t0 * pl.pieces[0];
    const long nbase = base0 + t1 * pl.pieces[1];
    const long full = (nbase / G) * G;
    const long rem = nbase - full;
    int item_len = pl.iters[0] / pl.pieces[0];
    if (t1 > 0) item_len = min(item_len, pl.iters[1] / pl.pieces[1]);
    long st = 1;
    if (rem > 0) {
      const long max_st = std::max<long>(1, std::min<long>(item_len / 16, kGemmPartialSlots / rem));
      if (tail_split > 0) {
        st = std::min<long>(tail_split, std::max(1, item_len / 16));
      } else {
        // pieces per tile of the last round: the least time on the busiest
        // workgroup, ceil(rem st / G) pieces of ceil(len / st) k-steps each
        // plus, for a split tile, about 4 + 4 st k-steps of writing and
        // summing fp32 partials per piece (measured: 336-tile and 384-tile
        // products at the 175B share, 3 and 2 pieces)
        long best = -1;
        for (long c = 1; c <= max_st; ++c) {
          const long t = (rem * c + G - 1) / G * ((item_len + c - 1) / c + (c > 1 ? 4 + 4 * c : 0));
          if (best < 0 || t < best) { best = t; st = c; }
        }
      }
      st = std::max<long>(std::min<long>(st, item_len), 1);
    }
    const long nitems = full + rem * st;
    const bool base_split = pl.pieces[0] > 1 || pl.pieces[1] > 1;
    const long slots = base_split ? nitems : (st > 1 ? nitems - full : 0);
    if (slots > kGemmPartialSlots && attempt == 0) continue;  // retry without base pieces
    if (slots > kGemmPartialSlots || nitems >= (1L << 30)) return hipErrorInvalidValue;
    pl.base0 = static_cast<int>(base0);
    pl.full_items = static_cast<int>(full);
    pl.tail_split = static_cast<int>(st);
    pl.nitems = static_cast<int>(nitems);
    pl.full_slots = base_split ? static_cast<int>(full) : 0;
    *out = pl;
    *grid_out = static_cast<int>(std::min<long>(G, nitems));
    return hipSuccess;
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_tiles(int M, int N) { return tiles_of(M, N); }

int device_compute_units() { return device_cus(); }

hipError_t launch_zero_i32(int* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gemm_group(const GemmProblem* probs, int nprob, Major a_major,
                             Major b_major, EpiMode mode, const GemmScratch& ws,
                             hipStream_t s, bool f16_prob0) {
  SkPlan pl;
  int grid = 0;
  const hipError_t e = build_plan(probs, nprob, a_major, b_major, ws, 0, &pl, &grid);
  if (e != hipSuccess) return e;
  if (f16_prob0) {
    // fp16 problem 0: the [q | k] product beside [v | FC1] (eight waves)
    if (a_major != KMAJOR || b_major != OUTER_MAJOR) return hipErrorInvalidValue;
    if (mode == EPI_QKV_GELU)
      return launch_plan<KMAJOR, OUTER_MAJOR, EPI_QKV_GELU, true>(pl, grid, s);
    if (mode == EPI_QKV_SWIGLU)
      return launch_plan<KMAJOR, OUTER_MAJOR, EPI_QKV_SWIGLU, true>(pl, grid, s);
    return hipErrorInvalidValue;
  }
  if (a_major == KMAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_QKV_GELU) return launch_plan<KMAJOR, OUTER_MAJOR, EPI_QKV_GELU>(pl, grid, s);
    if (mode == EPI_QKV_SWIGLU)
      return launch_plan<KMAJOR, OUTER_MAJOR, EPI_QKV_SWIGLU>(pl, grid, s);
    if (mode == EPI_RESIDUAL) return launch_plan<KMAJOR, OUTER_MAJOR, EPI_RESIDUAL>(pl, grid, s);
  } else if (a_major == KMAJOR && b_major == KMAJOR) {
    if (mode == EPI_DGELU) return launch_plan<KMAJOR, KMAJOR, EPI_DGELU>(pl, grid, s);
    if (mode == EPI_DSWIGLU) return launch_plan<KMAJOR, KMAJOR, EPI_DSWIGLU>(pl, grid, s);
    if (mode == EPI_STORE2_COLS) return launch_plan<KMAJOR, KMAJOR, EPI_STORE2_COLS>(pl, grid, s);
  } else if (a_major == OUTER_MAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_STORE2_ROWS) return launch_plan<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_ROWS>(pl, grid, s);
    if (mode == EPI_STORE2_COLS) return launch_plan<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_COLS>(pl, grid, s);
  }
  // the combinations the layer uses; anything else is a library bug
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_fp8(const GemmProblem& prob, Fp8Format fa, const float* amax_a,
                           Fp8Format fb, const float* amax_b, EpiMode mode,
                           const GemmScratch& ws, hipStream_t s) {
  // 16-byte rows of 8-bit elements; both scales present
  if (prob.A.ld0 % 16 != 0 || prob.A.ld1 % 16 != 0 || prob.B.ld0 % 16 != 0 ||
      prob.B.ld1 % 16 != 0 || amax_a == nullptr || amax_b == nullptr)
    return hipErrorInvalidValue;
  SkPlan pl;
  int grid = 0;
  const hipError_t e = build_plan(&prob, 1, KMAJOR, KMAJOR, ws, 0, &pl, &grid, 2 * BK);
  if (e != hipSuccess) return e;
  pl.amax_a = amax_a;
  pl.amax_b = amax_b;
  const int fmt = 1 + fa + 2 * fb;
  if (fmt == 1 && mode == EPI_QKV_GELU) return launch_plan_fp8<EPI_QKV_GELU, 1>(pl, grid, s);
  if (fmt == 1 && mode == EPI_RESIDUAL) return launch_plan_fp8<EPI_RESIDUAL, 1>(pl, grid, s);
  if (fmt == 2 && mode == EPI_DGELU) return launch_plan_fp8<EPI_DGELU, 2>(pl, grid, s);
  if (fmt == 2 && mode == EPI_STORE2_COLS) return launch_plan_fp8<EPI_STORE2_COLS, 2>(pl, grid, s);
  if (fmt == 3 && mode == EPI_STORE2_ROWS) return launch_plan_fp8<EPI_STORE2_ROWS, 3>(pl, grid, s);
  if (fmt == 3 && mode == EPI_STORE2_COLS) return launch_plan_fp8<EPI_STORE2_COLS, 3>(pl, grid, s);
  return hipErrorInvalidValue;  // a combination the FP8 layer does not use
}

hipError_t launch_gemm_mx(const GemmProblem& prob, Fp8Format fa, const MxScales& sa,
                          Fp8Format fb, const MxScales& sb, EpiMode mode,
                          const GemmScratch& ws, hipStream_t s) {
  // 16-byte rows of 8-bit elements, whole 128-wide k-steps, scale words for
  // every row of both operands
  if (prob.A.ld0 % 16 != 0 || prob.A.ld1 % 16 != 0 || prob.B.ld0 % 16 != 0 ||
      prob.B.ld1 % 16 != 0 || prob.K % (2 * BK) != 0 || sa.p == nullptr || sb.p == nullptr ||
      sa.ld < prob.M || sb.ld < prob.N || sa.ld % 128 != 0 || sb.ld % 128 != 0)
    return hipErrorInvalidValue;
  const size_t ks = static_cast<size_t>(prob.K) / (2 * BK);
  if (ks * sa.ld * 4 >= (1UL << 31) || ks * sb.ld * 4 >= (1UL << 31)) return hipErrorInvalidValue;
  SkPlan pl;
  int grid = 0;
  const hipError_t e = build_plan(&prob, 1, KMAJOR, KMAJOR, ws, 0, &pl, &grid, 2 * BK);
  if (e != hipSuccess) return e;
  pl.scale_a = sa.p;
  pl.scale_b = sb.p;
  pl.scale_lda = sa.ld;
  pl.scale_ldb = sb.ld;
  pl.scale_bytes_a = static_cast<uint32_t>(ks * sa.ld * 4);
  pl.scale_bytes_b = static_cast<uint32_t>(ks * sb.ld * 4);
  const int fmt = 1 + fa + 2 * fb;
  if (fmt == 1 && mode == EPI_QKV_GELU) return launch_plan_fp8<EPI_QKV_GELU, 1, true>(pl, grid, s);
  if (fmt == 1 && mode == EPI_RESIDUAL) return launch_plan_fp8<EPI_RESIDUAL, 1, true>(pl, grid, s);
  if (fmt == 2 && mode == EPI_DGELU) return launch_plan_fp8<EPI_DGELU, 2, true>(pl, grid, s);
  if (fmt == 2 && mode == EPI_STORE2_COLS) return launch_plan_fp8<EPI_STORE2_COLS, 2, true>(pl, grid, s);
  if (fmt == 3 && mode == EPI_STORE2_ROWS) return launch_plan_fp8<EPI_STORE2_ROWS, 3, true>(pl, grid, s);
  if (fmt == 3 && mode == EPI_STORE2_COLS) return launch_plan_fp8<EPI_STORE2_COLS, 3, true>(pl, grid, s);
  return hipErrorInvalidValue;  // a combination the FP8 layer does not use
}

hipError_t launch_gemm(int M, int N, int K, const Operand& A, Major a_major,
                       const Operand& B, Major b_major, EpiMode mode,
                       const Epilogue& e, const GemmScratch& ws, hipStream_t s) {
  GemmProblem p;
  p.M = M; p.N = N; p.K = K; p.A = A; p.B = B; p.epi = e;
  return launch_gemm_group(&p, 1, a_major, b_major, mode, ws, s);
}

}  // namespace ptb
