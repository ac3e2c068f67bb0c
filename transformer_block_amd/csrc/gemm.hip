// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16) with LDS-staged,
// double-buffered tiles and fused epilogues.
//
// One kernel template covers the six matrix products of the Parallel
// Transformer Block layer (MegaScale reading notes, section 1.1, eq (4); fused
// QKV projection, section 1.3; MLP Y = GeLU(XA)B, Megatron-LM tensor-parallel
// explainer, section 2.1):
//   forward   [QKV | FC1]:  a [T,h]      x [W_qkv | W_fc1]      -> qkv, u, GeLU(u)
//             [O ; FC2]:    [c | g]      x [W_o ; W_fc2]  + x   -> y
//   backward  dgrad:        dy x [W_o ; W_fc2]^T  (x GeLU'(u))  -> dc, du
//                           dZ x [W_qkv | W_fc1]^T              -> da (fp32)
//             wgrad:        [c | g]^T x dy                      -> dW_o, dW_fc2
//                           a^T x dZ                            -> dW_qkv, dW_fc1
// Concatenations are addressed in place (two-segment operands), never copied.
//
// Tiling: a 256-thread workgroup (4 waves of 64 lanes, 2 x 2) owns a BM x BN
// tile of C and walks K in steps of 64.  Both operands are staged in LDS as
// rows of 64 k-values (128 bytes, XOR-swizzled) so that every MFMA fragment is
// one 16-byte LDS read.  An operand whose k index is not contiguous in memory
// (weights in the forward, activations in the weight gradients) is loaded
// 16 bytes at a time along its contiguous dimension and transposed in
// registers on the way into LDS.  The next K tile is fetched into registers
// while the current one feeds the matrix cores.  Tiles are handed out
// XCD-aware: consecutive workgroups go round-robin over the 8 XCDs, so the
// tile index is remapped to give each XCD a contiguous, L2-friendly group of
// tiles.
#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int BK = 64;

// Buffer resource over one operand segment: reads at or beyond `bytes` return
// zero, which covers ragged row counts and the k tail without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const u16* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Segment of the k-tile starting at k0 and k0 relative to that segment.
// Split points are multiples of 64 (= BK), so a k-tile never straddles one.
__device__ __forceinline__ void k_segment(const Operand& op, int k0, int& seg, int& krel) {
  seg = (op.split_on_k && k0 >= op.split) ? 1 : 0;
  krel = seg ? k0 - op.split : k0;
}

template <int R, int MAJ>
struct TileLoader;

// k contiguous in memory: thread t loads chunk (t & 7) of rows (t >> 3) + 32*i;
// the 16-byte chunks go straight to LDS.  A wave's rows for one i lie in one
// aligned block of 32, so the segment (split points are multiples of 32) is
// uniform across the wave.
template <int R>
struct TileLoader<R, KMAJOR> {
  static constexpr int NCH = R / 32;
  uint4 v[NCH];
  int off0[NCH], off1[NCH];  // byte offset of the row start in either segment
  int oseg[NCH];             // segment of the row when the split is on the outer index

  __device__ __forceinline__ void init(const Operand& op, int r0, int tid) {
    const int rr = tid >> 3, c = tid & 7;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = r0 + rr + 32 * i;
      int sg = (!op.split_on_k && r >= op.split) ? 1 : 0;
      sg = __builtin_amdgcn_readfirstlane(sg);
      oseg[i] = sg;
      const int r1 = op.split_on_k ? r : r - op.split;
      off0[i] = (r * op.ld0 + c * 8) * 2;
      off1[i] = (r1 * op.ld1 + c * 8) * 2;
    }
  }
  __device__ __forceinline__ void load(const Operand& op, __amdgpu_buffer_rsrc_t rs0,
                                       __amdgpu_buffer_rsrc_t rs1, int k0) {
    int kseg, krel;
    k_segment(op, k0, kseg, krel);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int sg = op.split_on_k ? kseg : oseg[i];
      v[i] = sg ? load16(rs1, off1[i] + krel * 2) : load16(rs0, off0[i] + krel * 2);
    }
  }
  __device__ __forceinline__ void store(u16* lds, int tid) const {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = rr + 32 * i;
      *reinterpret_cast<uint4*>(lds + r * BK + ((c ^ swz128(r)) << 3)) = v[i];
    }
  }
};

// Outer index contiguous in memory: each thread loads a KS x 8 block (KS
// k-rows of 8 consecutive outer indices) and writes it transposed.  Wave w
// owns outer indices [R/4*w, R/4*(w+1)) of the tile, an aligned block of 64
// (R = 256) or 32 (R = 128), so its segment is uniform.
template <int R>
struct TileLoader<R, OUTER_MAJOR> {
  static constexpr int KS = R / 32;   // k rows per thread: 8 (R = 256) or 4 (R = 128)
  static constexpr int GPW = R / 32;  // 8-wide outer groups per wave
  uint32_t w[KS][4];
  int base0, base1;  // byte offset of (k = kg*KS, outer group) in either segment
  int oseg;

  __device__ __forceinline__ static void coords(int tid, int& rg, int& kg) {
    const int wv = tid >> 6, l = tid & 63;
    rg = GPW * wv + (l % GPW);
    kg = l / GPW;
  }
  __device__ __forceinline__ void init(const Operand& op, int r0, int tid) {
    int rg, kg;
    coords(tid, rg, kg);
    const int outer = r0 + rg * 8;
    int sg = (!op.split_on_k && outer >= op.split) ? 1 : 0;
    sg = __builtin_amdgcn_readfirstlane(sg);
    oseg = sg;
    const int o1 = op.split_on_k ? outer : outer - op.split;
    base0 = (kg * KS * op.ld0 + outer) * 2;
    base1 = (kg * KS * op.ld1 + o1) * 2;
  }
  __device__ __forceinline__ void load(const Operand& op, __amdgpu_buffer_rsrc_t rs0,
                                       __amdgpu_buffer_rsrc_t rs1, int k0) {
    int kseg, krel;
    k_segment(op, k0, kseg, krel);
    const int sg = op.split_on_k ? kseg : oseg;
    const int ld = sg ? op.ld1 : op.ld0;
    const int base = sg ? base1 : base0;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 t = load16(sg ? rs1 : rs0, base + (krel + kk) * ld * 2);
      w[kk][0] = t.x; w[kk][1] = t.y; w[kk][2] = t.z; w[kk][3] = t.w;
    }
  }
  __device__ __forceinline__ void store(u16* lds, int tid) const {
    int rg, kg;
    coords(tid, rg, kg);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = rg * 8 + j;
      uint32_t o[KS / 2];
#pragma unroll
      for (int p = 0; p < KS / 2; ++p) {
        const uint32_t a = w[2 * p][j >> 1], b = w[2 * p + 1][j >> 1];
        o[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      if constexpr (KS == 8) {
        *reinterpret_cast<uint4*>(lds + row * BK + ((kg ^ swz128(row)) << 3)) =
            make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        *reinterpret_cast<uint2*>(lds + row * BK + (((kg >> 1) ^ swz128(row)) << 3) +
                                  ((kg & 1) << 2)) = make_uint2(o[0], o[1]);
      }
    }
  }
};

__device__ __forceinline__ bf16x8 frag(const u16* lds, int row, int chunk) {
  return as_bf16x8(
      *reinterpret_cast<const uint4*>(lds + row * BK + ((chunk ^ swz128(row)) << 3)));
}

// ---- epilogue
// Each wave stages one 32 x 32 fp32 accumulator block at a time in a private
// LDS region (row stride 36 floats), then lane l takes row l/2, columns
// 16*(l%2) .. +15 of the block: the epilogue math sees 16 consecutive columns
// and writes them with 16- and 32-byte vector stores.
constexpr int EPI_LD = 36;

__device__ __forceinline__ void store16bf(u16* p, const float* v) {
  uint4 a, b;
  a.x = pack2bf(v[0], v[1]);   a.y = pack2bf(v[2], v[3]);
  a.z = pack2bf(v[4], v[5]);   a.w = pack2bf(v[6], v[7]);
  b.x = pack2bf(v[8], v[9]);   b.y = pack2bf(v[10], v[11]);
  b.z = pack2bf(v[12], v[13]); b.w = pack2bf(v[14], v[15]);
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
template <int MODE>
__device__ __forceinline__ void epi_row16(const Epilogue& e, int region, int r, int c, float* v) {
  if constexpr (MODE == EPI_QKV_GELU) {
    const int gc = c + e.col_base;
    if (region == 0) {
      float lo[16];
      uint4 a, b;
      uint32_t* w = reinterpret_cast<uint32_t*>(&a);
      uint32_t* x = reinterpret_cast<uint32_t*>(&b);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = pack2bf(v[2 * i], v[2 * i + 1]);
        x[i] = pack2bf(v[8 + 2 * i], v[9 + 2 * i]);
        lo[2 * i] = v[2 * i] - lo_bf(w[i]);
        lo[2 * i + 1] = v[2 * i + 1] - hi_bf(w[i]);
        lo[8 + 2 * i] = v[8 + 2 * i] - lo_bf(x[i]);
        lo[9 + 2 * i] = v[9 + 2 * i] - hi_bf(x[i]);
      }
      uint4* o = reinterpret_cast<uint4*>(e.o0 + r * e.ld0 + gc);
      o[0] = a;
      o[1] = b;
      store16bf(e.o3 + r * e.ld3 + gc, lo);
    } else if (region == 1) {
      store16bf(e.o0 + r * e.ld0 + gc, v);
    } else {
      const int cc = gc - e.split;
      store16bf(e.o1 + r * e.ld1 + cc, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = gelu_f(v[i]);
      store16bf(e.o2 + r * e.ld1 + cc, v);
    }
  } else if constexpr (MODE == EPI_RESIDUAL) {
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
  if constexpr (MODE == EPI_QKV_GELU) {
    const int g = cb + e.col_base;
    return g < e.lo_cols ? 0 : (g < e.split ? 1 : 2);
  } else if constexpr (MODE == EPI_DGELU || MODE == EPI_STORE2_COLS) {
    return cb < e.split ? 0 : 1;
  } else if constexpr (MODE == EPI_STORE2_ROWS) {
    return r0 < e.split ? 0 : 1;
  } else {
    return 0;
  }
}

// Scheduling groups (instruction classes for __builtin_amdgcn_sched_group_barrier).
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;

struct GemmBatch {
  GemmProblem p[2];
  int tiles0;  // tiles of problem 0; the rest of the grid belongs to problem 1
};

template <int BM, int BN>
__host__ __device__ inline int tile_count(const GemmProblem& p) {
  return ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
}

template <int BM, int BN, int AMAJ, int BMAJ, int MODE>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmBatch batch) {
  constexpr int WM = BM / 2, WN = BN / 2;  // per-wave tile
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int NMF = FM * FN;             // MFMAs per k-step per wave
  constexpr int NFR = FM + FN;             // fragment reads per k-step per wave
  __shared__ __attribute__((aligned(16))) u16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile index.  Consecutive workgroups go round-robin over the 8 XCDs
  // (each with its own L2), and an XCD runs its workgroups in order.  XCD x
  // gets an equal share of each problem's tiles, each share a contiguous range
  // (L2 reuse), problem 0 first (its tiles may be longer: longest first).
  int pid;
  bool second;
  {
    const int nall = gridDim.x, t0 = batch.tiles0;
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int base = nall / 8, rem = nall % 8;
    const int before = xcd * base + min(xcd, rem);     // workgroups on XCDs < xcd
    const int cnt = base + (xcd < rem ? 1 : 0);         // workgroups on this XCD
    // problem-0 tiles in proportion to the XCD's workgroups: n0 <= cnt, and
    // over all XCDs each tile of either problem is taken exactly once
    const int s0 = static_cast<int>(static_cast<long long>(t0) * before / nall);
    const int n0 = static_cast<int>(static_cast<long long>(t0) * (before + cnt) / nall) - s0;
    second = loc >= n0;
    pid = second ? (before - s0) + (loc - n0) : s0 + loc;
  }
  const GemmProblem& P = second ? batch.p[1] : batch.p[0];
  const int M = P.M, N = P.N, K = P.K;
  const Operand& A = P.A;
  const Operand& B = P.B;
  const Epilogue& epi = P.epi;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  constexpr int GM = 8;
  const int span = GM * tiles_n;
  const int first_m = (pid / span) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % span) % gsz;
  const int tn = (pid % span) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  TileLoader<BM, AMAJ> la;
  TileLoader<BN, BMAJ> lb;
  la.init(A, m0, tid);
  lb.init(B, n0, tid);
  const __amdgpu_buffer_rsrc_t ra0 = make_rsrc(A.p0, A.bytes0), ra1 = make_rsrc(A.p1, A.bytes1);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B.p0, B.bytes0), rb1 = make_rsrc(B.p1, B.bytes1);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lrow = lane & 31, lk = lane >> 5;
  const int arow = wm * WM + lrow, brow = wn * WN + lrow;
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const u16* As, int ks, int slot) {
    const u16* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[slot][i] = frag(As, arow + i * 32, ks * 2 + lk);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[slot][j] = frag(Bs, brow + j * 32, ks * 2 + lk);
  };
  auto mfma_step = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[slot][i], fb[slot][j], acc[i][j]);
  };

  // Prologue: tile 0 into LDS buffer 0, first fragments into registers.
  const int nk = (K + BK - 1) / BK;
  la.load(A, ra0, ra1, 0);
  lb.load(B, rb0, rb1, 0);
  la.store(smem, tid);
  lb.store(smem + BM * BK, tid);
  __syncthreads();
  read_frags(smem, 0, 0);

  // Main loop.  Iteration kt computes tile kt from LDS buffer kt&1 while tile
  // kt+1 streams in: global -> registers at the start, registers -> the other
  // LDS buffer after k-step 2, one barrier before k-step 3, after which the
  // first fragments of tile kt+1 are read under the MFMAs of k-step 3.
  // Fragments are double-buffered in registers, so the LDS reads of k-step
  // s+1 are in flight while the MFMAs of k-step s run.  The prefetch past the
  // last tile reads zeros (buffer bounds) and is never used.
  for (int kt = 0; kt < nk; ++kt) {
    u16* cur = smem + (kt & 1) * STAGE;
    u16* nxt = smem + ((kt & 1) ^ 1) * STAGE;
    la.load(A, ra0, ra1, (kt + 1) * BK);
    lb.load(B, rb0, rb1, (kt + 1) * BK);
    read_frags(cur, 1, 1);
    mfma_step(0);
    read_frags(cur, 2, 0);
    mfma_step(1);
    read_frags(cur, 3, 1);
    mfma_step(0);
    la.store(nxt, tid);
    lb.store(nxt + BM * BK, tid);
    // interleave: global loads and LDS reads between the MFMAs of k-steps 0-2,
    // the LDS writes of the next tile after them
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (i < NFR) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (i < NFR) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (i < NFR) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 64, 0);
    __syncthreads();
    read_frags(nxt, 0, 0);
    mfma_step(1);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 1);
      if (i < NFR) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 1);
    }
  }

  // ---- epilogue, one 32 x 32 block at a time through LDS
  __syncthreads();
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * EPI_LD;
  const int er = lane >> 1, ec = (lane & 1) * 16;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r0 = m0 + wm * WM + i * 32, cb = n0 + wn * WN + j * 32;
#pragma unroll
      for (int q = 0; q < 16; ++q) ep[((q >> 2) * 8 + lk * 4 + (q & 3)) * EPI_LD + lrow] = acc[i][j][q];
      __builtin_amdgcn_wave_barrier();
      float v[16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 x = *reinterpret_cast<const float4*>(ep + er * EPI_LD + ec + 4 * t);
        v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
      }
      __builtin_amdgcn_wave_barrier();
      const int region = __builtin_amdgcn_readfirstlane(epi_region<MODE>(epi, r0, cb));
      const int r = r0 + er;
      if (cb < N && r < M) epi_row16<MODE>(epi, region, r, cb + ec, v);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int BM, int BN, int AMAJ, int BMAJ, int MODE>
hipError_t launch_tiles(const GemmProblem* probs, int nprob, hipStream_t s) {
  GemmBatch b;
  b.p[0] = probs[0];
  b.p[1] = nprob > 1 ? probs[1] : probs[0];
  b.tiles0 = tile_count<BM, BN>(probs[0]);
  const int nt = b.tiles0 + (nprob > 1 ? tile_count<BM, BN>(probs[1]) : 0);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AMAJ, BMAJ, MODE>), dim3(nt), dim3(256), 0, s, b);
  return hipGetLastError();
}

template <int AMAJ, int BMAJ, int MODE>
hipError_t launch_sized(const GemmProblem* probs, int nprob, hipStream_t s) {
  long big = 0;
  for (int i = 0; i < nprob; ++i) big += tile_count<256, 256>(probs[i]);
  if (big >= 192) return launch_tiles<256, 256, AMAJ, BMAJ, MODE>(probs, nprob, s);
  return launch_tiles<128, 128, AMAJ, BMAJ, MODE>(probs, nprob, s);
}

}  // namespace

hipError_t launch_gemm_group(const GemmProblem* probs, int nprob, Major a_major,
                             Major b_major, EpiMode mode, hipStream_t s) {
  if (nprob < 1 || nprob > 2) return hipErrorInvalidValue;
  for (int i = 0; i < nprob; ++i)
    if (probs[i].M <= 0 || probs[i].N <= 0) return hipErrorInvalidValue;
  // The combinations used by the layer; anything else is a library bug.
  if (a_major == KMAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_QKV_GELU) return launch_sized<KMAJOR, OUTER_MAJOR, EPI_QKV_GELU>(probs, nprob, s);
    if (mode == EPI_RESIDUAL) return launch_sized<KMAJOR, OUTER_MAJOR, EPI_RESIDUAL>(probs, nprob, s);
  } else if (a_major == KMAJOR && b_major == KMAJOR) {
    if (mode == EPI_DGELU) return launch_sized<KMAJOR, KMAJOR, EPI_DGELU>(probs, nprob, s);
    if (mode == EPI_F32) return launch_sized<KMAJOR, KMAJOR, EPI_F32>(probs, nprob, s);
  } else if (a_major == OUTER_MAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_STORE2_ROWS) return launch_sized<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_ROWS>(probs, nprob, s);
    if (mode == EPI_STORE2_COLS) return launch_sized<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_COLS>(probs, nprob, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int M, int N, int K, const Operand& A, Major a_major,
                       const Operand& B, Major b_major, EpiMode mode,
                       const Epilogue& e, hipStream_t s) {
  GemmProblem p;
  p.M = M; p.N = N; p.K = K; p.A = A; p.B = B; p.epi = e;
  return launch_gemm_group(&p, 1, a_major, b_major, mode, s);
}

}  // namespace ptb
