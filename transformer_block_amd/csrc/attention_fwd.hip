// Sliding-window causal flash attention, forward pass, for gfx950.  What is
// computed and the matrix-core mapping are described in attention.hip.
#include "attention_common.h"

namespace ptb {
namespace {

// ------------------------------------------------------------------ forward
// Stage of BKF keys in LDS, filled by DMA one tile ahead of the matrix cores,
// two stages: fp16 K row-major (read by row_frag), bf16 V in the outer layout
// with its rows in the S^T accumulator's key order (read transposed).
constexpr float kStale = 8.0f;

// Keys per LDS tile and stages of the ring: 32 keys per tile, FNST stages
// (FNST - 1 tiles in flight while one is computed; 16 KB each for D = 128),
// so that one workgroup's softmax and barrier waits run beside another's
// MFMAs.  One stage of lead is not enough once each logit is a single fp16
// MFMA: a tile's compute is then shorter than the latency of its loads.  Two
// builds: four stages with two workgroups per CU, and three stages with
// three (48 KB of LDS and at most 168 registers each); more workgroups per CU
// hide more latency (+13% forward throughput on the 5120-hidden stack) but
// make each item slower (the 175B share's few long rows: 40 -> 47 us), so
// the launcher picks by the dispatch model (plan_rows).
constexpr int BKF = 32;
constexpr int KB = BKF / 32;  // 32 x 32 S^T blocks per tile
// time per tile of a workgroup with three per CU, relative to two per CU
// (measured: 1.5 x the workgroups per CU for 1.13 x the throughput)
constexpr double kFwd3TileCost = 1.33;

template <int D, int FNST>
__global__ __launch_bounds__(256, FNST == 4 ? 2 : 3) void attn_fwd_kernel(const u16* __restrict__ qkv,
                                                       const u16* __restrict__ qk16,
                                                       u16* __restrict__ cout,
                                                       float* __restrict__ lse, int s, int n,
                                                       int window, int nqt, RowSplit rs) {
  constexpr int NKS = D / 16, ND = D / 32;
  constexpr int OPB = BKF * D;  // u16 elements of one operand's tile
  constexpr int STG = 2 * OPB;  // one stage: K (fp16), V (bf16)
  __shared__ __attribute__((aligned(1024))) u16 kv[FNST * STG];
  __shared__ int arrival;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const RowBlock rb = row_block(rs, n);
  const RowItem item = decode_row_item<true>(rb.item, nqt, s, window, rs.ch);
  if (item.nchunks == 0) return;
  const int qt = item.row;
  const int hd = rb.hd, bi = rb.bi;
  const int hl = n * D, ld = 3 * hl;
  const u16* Qh = qk16 + static_cast<size_t>(bi) * s * (2 * hl) + hd * D;  // fp16
  const u16* Kh = Qh + hl;
  const u16* Vg = qkv + static_cast<size_t>(bi) * s * ld + hd * D + 2 * hl;  // bf16
  const int q0 = qt * BQ, qw0 = q0 + wave * 32, qi = qw0 + l32;

  const int kv_begin = item.span.begin;
  const int kv_end = item.span.end;
  TileDma<D, BKF, false> dk;
  TileDma<D, BKF, true> dv;
  constexpr int LPT = TileDma<D, BKF, false>::LPW + TileDma<D, BKF, true>::LPW;  // loads/tile/wave
  dk.init(Kh, 2 * hl, s, wave, lane);
  dv.init(Vg, ld, s, wave, lane);
  const uint32_t kv_lds = __builtin_amdgcn_readfirstlane(lds_address(kv));
  // tile kt0 into ring stage st, or (kt0 past the span) loads that only keep
  // the count of loads in flight constant
  auto issue = [&](int st, int kt0) {
    const uint32_t lds = kv_lds + st * (STG * 2);
    if (kt0 < kv_end) {
      dk.issue(lds, kt0, wave);
      dv.issue(lds + OPB * 2, kt0, wave);
    } else {
      dk.issue_none(lds, wave);
      dv.issue_none(lds + OPB * 2, wave);
    }
  };
  // The row's queries go by DMA too, first, into the ring's last two stages
  // (four tiles of 32 rows, 32 KB), then the first FNST - 2 key tiles; the
  // wave waits for the queries only, reads its fragments, and after a
  // barrier the stage they used receives key tile FNST - 2.  The first tile's
  // products can then start while the later tiles are still on their way.
  static_assert(BQ == 4 * BKF && FNST >= 3, "the queries fill two ring stages");
  {
    TileDma<D, BKF, false> dq;
    dq.init(Qh, 2 * hl, s, wave, lane);
    const uint32_t q_lds = kv_lds + (FNST - 2) * (STG * 2);
#pragma unroll
    for (int t = 0; t < BQ / BKF; ++t) dq.issue(q_lds + t * (OPB * 2), q0 + t * BKF, wave);
  }
#pragma unroll
  for (int i = 0; i < FNST - 2; ++i) issue(i, kv_begin + i * BKF);
  wait_vm_lds<(FNST - 2) * LPT>();  // this wave's query loads landed
  __syncthreads();                  // every wave's
  bf16x8 qf[NKS];  // fp16 query fragments (B operand of S^T = K Q^T); rows past s are zeros
  {
    const u16* q_w = kv + (FNST - 2) * STG + wave * OPB;  // this wave's 32 queries
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = row_frag<D>(q_w, l32, ks * 2 + g);
  }
  wait_vm_lds<63>();  // (LDS only) every fragment read here ...
  __syncthreads();    // ... and in every wave before the stage is refilled
  issue(FNST - 2, kv_begin + (FNST - 2) * BKF);

  // Running max m is kept in scaled (log2) units: p = exp2(logit * sc - m).
  const float sc = kLog2e / sqrtf(static_cast<float>(D));
  float m = -INFINITY, l = 0.0f;
  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;

  int stage = 0;
  for (int kt0 = kv_begin; kt0 < kv_end; kt0 += BKF) {
    // this wave's loads of tile kt0 landed (FNST - 2 later tiles' may still
    // be in flight: loads complete in order)
    wait_vm_lds<(FNST - 2) * LPT>();
    __syncthreads();  // every wave's; the stage read last iteration is free again
    issue(stage == 0 ? FNST - 1 : stage - 1, kt0 + (FNST - 1) * BKF);
    const u16* k_lds = kv + stage * STG;
    const u16* v_lds = k_lds + OPB;
    stage = stage == FNST - 1 ? 0 : stage + 1;

    const bool any = qw0 < s && qw0 + 31 >= kt0 && qw0 - (kt0 + BKF - 1) < window;
    if (!any) continue;
    const bool full = kt0 + BKF - 1 <= qw0 && qw0 + 31 - kt0 < window && kt0 + BKF <= s;

    // each chain's first product takes a literal zero accumulator
    const f32x16 zero = {};
    f32x16 st[KB];
    // S^T = K Q^T in fp16, one MFMA per 16-wide k-step: the tile's key
    // fragments are all read first, the products chained after them
    bf16x8 fk[KB][NKS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) fk[kb][ks] = row_frag<D>(k_lds, kb * 32 + l32, ks * 2 + g);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        st[kb] = mfma32x32x16_f16(fk[kb][ks], qf[ks], ks == 0 ? zero : st[kb]);
    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[kb][e]);
    } else {
      // a tile on the diagonal or the window's edge: keep keys in [lo, hi]
      // of this lane's query, as offsets from the lane's first key
      asm volatile("; masked key tile");  // keeps this path a real branch
      const int base = kt0 + g * 4;
      const int lo = max(qi - window + 1, 0) - base;
      const int hi = min(qi, s - 1) - base;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kb * 32 + (e >> 2) * 8 + (e & 3);
          if (off < lo || off > hi) st[kb][e] = -INFINITY;
          mx = fmaxf(mx, st[kb][e]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // The reference point m of the exponentials moves only when some query
    // of the wave sees a logit more than kStale (log2 units) above it: below
    // that, p = exp2(logit * sc - m) <= 2^kStale stays well inside fp32 and
    // bf16 range, and o and l stay consistent with the same m, so the final
    // o / l and lse = m + log2 l do not depend on when m moved.
    const float mcand = mx * sc;
    if (__builtin_amdgcn_ballot_w64(mcand > m + kStale) != 0) {
      const float mnew = fmaxf(m, mcand);
      // a lane with no key yet keeps m = -inf: its alpha is exp2(-inf) = 0
      const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.0f : mnew));
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m = mnew;
    }
    const float msafe = (m == -INFINITY) ? 0.0f : m;
    float rsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[kb][e], sc, -msafe));
        st[kb][e] = p;
        rsum += p;
      }
    l += rsum;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const bf16x8 pb = pack8(st[kb], e2 * 8);
#pragma unroll
        for (int db = 0; db < ND; ++db)
          o[db] = mfma32x32x16(frag_outer<BKF>(v_lds, db * 32, kb * 2 + e2, lane), pb, o[db]);
      }
  }

  // the trailing loads (beyond the span) write zeros into the ring: every
  // one of them lands before the workgroup can finish and its LDS be reused
  wait_vm_lds<0>();

  if (item.nchunks > 1) {
    // A chunk of a split row: store o, m and l (device scope), count in; the
    // last chunk to arrive merges all of them, in chunk order.
    constexpr int PER_SLOT = BQ * D + 2 * 256;
    const size_t row_id = (static_cast<size_t>(bi) * n + hd) * nqt + qt;
    const size_t slot0 = (static_cast<size_t>(bi) * n + hd) * rs.split_slots;
    const int first_slot = item.slot - item.chunk;
    {
      float* pp = rs.partials + (slot0 + item.slot) * PER_SLOT;
      const __amdgpu_buffer_rsrc_t pr = dev_rsrc(pp, PER_SLOT);
#pragma unroll
      for (int db = 0; db < ND; ++db) st16_dev(pr, (wave * ND + db) * 1024, lane, o[db]);
      st_dev(pp + BQ * D + tid, m);
      st_dev(pp + BQ * D + 256 + tid, l);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) arrival = atomicAdd(rs.counters + row_id, 1);
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(arrival) != item.nchunks - 1) return;
    if (tid == 0) rs.counters[row_id] = 0;
    // Chunks in batches of MB, every load of a batch issued before its values
    // are used (each is a round trip to device memory): the maxima first,
    // then per batch the m and l, and the o partials summed in chunk order.
    // The two-per-CU build at d = 128 has the registers to keep this chunk's
    // own o (the bits it stored) instead of loading it back.
    constexpr int MB = 8;
    const int nch = item.nchunks;
    const float* ml0 = rs.partials + (slot0 + first_slot) * PER_SLOT + BQ * D + tid;
    float mm = -INFINITY;
    for (int c0 = 0; c0 < nch; c0 += MB) {
      float mv[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k)
        mv[k] = c0 + k < nch ? ld_dev(ml0 + static_cast<size_t>(c0 + k) * PER_SLOT) : -INFINITY;
#pragma unroll
      for (int k = 0; k < MB; ++k) mm = fmaxf(mm, mv[k]);
    }
    const float ms = (mm == -INFINITY) ? 0.0f : mm;
    constexpr bool OWN = FNST == 4 && D == 128;
    f32x16 own[OWN ? ND : 1];
    if constexpr (OWN) {
#pragma unroll
      for (int db = 0; db < ND; ++db) own[db] = o[db];
    }
    l = 0.0f;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += MB) {
      float mv[MB], lv[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const float* q = ml0 + static_cast<size_t>(c0 + k) * PER_SLOT;
        mv[k] = c0 + k < nch ? ld_dev(q) : 0.0f;
        lv[k] = c0 + k < nch ? ld_dev(q + 256) : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const int c = c0 + k;
        if (c >= nch) break;
        const float f = exp2f(mv[k] - ms);
        l += f * lv[k];
        const __amdgpu_buffer_rsrc_t pr =
            dev_rsrc(rs.partials + (slot0 + first_slot + c) * PER_SLOT, PER_SLOT);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          float x[16];
          if (OWN && c == item.chunk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = own[db][e];
          } else {
            ld16_dev(pr, (wave * ND + db) * 1024, lane, x);
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] += f * x[e];
        }
      }
    }
    m = mm;
  }

  const float lt = l + __shfl_xor(l, 32);
  if (qi < s) {
    const float inv = 1.0f / lt;
    u16* cg = cout + (static_cast<size_t>(bi) * s + qi) * hl + hd * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = db * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2*>(cg + d0) =
            make_uint2(pack2bf(o[db][jj * 4 + 0] * inv, o[db][jj * 4 + 1] * inv),
                       pack2bf(o[db][jj * 4 + 2] * inv, o[db][jj * 4 + 3] * inv));
      }
    if (g == 0) lse[(static_cast<size_t>(bi) * n + hd) * s + qi] = m + log2f(lt);
  }
}

template <int D>
hipError_t fwd_d(const u16* qkv, const u16* qk16, u16* c, float* lse, int b, int s, int n,
                 int window, const AttnScratch& sc, hipStream_t st) {
  const int nqt = (s + BQ - 1) / BQ;
  RowSplit rs2, rs3;
  int items2 = 0, items3 = 0;
  double t2 = 0.0, t3 = 0.0;
  hipError_t e = plan_rows<true>(b, s, n, window, nqt, BQ * D + 2 * 256,
                                 launch_slots(attn_fwd_kernel<D, 4>, sc), sc, &rs2, &items2, 1.0,
                                 &t2);
  if (e != hipSuccess) return e;
  e = plan_rows<true>(b, s, n, window, nqt, BQ * D + 2 * 256, launch_slots(attn_fwd_kernel<D, 3>, sc),
                      sc, &rs3, &items3, kFwd3TileCost, &t3);
  if (e != hipSuccess) return e;
  if (t3 < t2)
    hipLaunchKernelGGL((attn_fwd_kernel<D, 3>), dim3(items3 * rs3.nb), dim3(256), 0, st, qkv, qk16,
                       c, lse, s, n, window, nqt, rs3);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, 4>), dim3(items2 * rs2.nb), dim3(256), 0, st, qkv, qk16,
                       c, lse, s, n, window, nqt, rs2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fwd(const u16* qkv, const u16* qk16, u16* c, float* lse, int b,
                                int s, int n, int d, int window, const AttnScratch& sc,
                                hipStream_t st) {
  if (d == 128) return fwd_d<128>(qkv, qk16, c, lse, b, s, n, window, sc, st);
  if (d == 64) return fwd_d<64>(qkv, qk16, c, lse, b, s, n, window, sc, st);
  return hipErrorInvalidValue;
}


}  // namespace ptb
