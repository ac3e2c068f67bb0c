// Sliding-window causal flash attention for gfx950: what is computed, and the
// backward pass with the probabilities recomputed from the saved
// log-sum-exp (the forward pass is in attention_fwd.hip, the pieces both
// share in attention_common.h).
//
// What is computed (MegaScale reading notes, section 1.1, eq (5)-(6), and
// section 1.3): for each (batch, head) and query i, the keys j with
// 0 <= i - j < window, logits q_i . k_j / sqrt(d), a softmax over them and the
// weighted sum of v_j.  The s x s probability matrix never reaches HBM: the
// forward streams key tiles with an online softmax and stores only the
// per-query log-sum-exp; the backward recomputes P from it (selective
// recompute of the core attention, same notes section 1.3; Megatron tuning
// post, recompute section).  Key tiles that lie wholly outside every query's
// window are never visited, so the work is O(s * w), not O(s^2).
//
// Matrix-core mapping.  Every contraction is a 32x32x16 MFMA: fp16 for the
// logits and the products with dS, bf16 for the rest.  The forward computes S^T = K Q^T so that each lane owns one query column: the
// row max and row sum of the online softmax are lane-local plus one exchange
// with the lane 32 apart, and O^T = V^T P^T reuses the S^T accumulator
// registers directly as the B operand (the key order inside a 16-key step is
// permuted identically on both operands, which leaves the sum unchanged).
// The forward's key tiles reach LDS by DMA one tile ahead, and V^T is read
// from the row-major V tile by the transposing LDS read (the permutation is
// applied to V's rows as they are loaded).  The backward splits into
// a key-parallel kernel for dK, dV (S = Q K^T, lane = key) and a
// query-parallel kernel for dQ (S^T, lane = query), so no atomics are needed
// and results are deterministic.
//
// Logit precision.  q and k arrive in fp16 (10 mantissa bits, from an fp32
// product of the fp16 copies of LN(x) and of the q, k weight columns), and
// every logit is one fp16 matrix-core product.  With the large logits of wide
// layers a bf16 rounding of LN(x), q or k would shift every logit by a few
// thousandths, which the softmax turns into a relative error of the same size
// in the output and, through dS, in the gradients of q and k; fp16 cuts that
// shift by 8x at the same cost as bf16.  dS goes to fp16 as well for the
// products with k and q (dQ = dS K, dK = dS^T Q); P and dO stay bf16 (dV =
// P^T dO, dP = dO V^T, O = P V).
#include "attention_common.h"

namespace ptb {
namespace {

// ------------------------------------------------- delta = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const u16* __restrict__ dc,
                                                         const u16* __restrict__ c,
                                                         float* __restrict__ delta, int T,
                                                         int s, int n) {
  constexpr int LPI = D / 8;  // lanes per (token, head)
  const int item = (blockIdx.x * 256 + threadIdx.x) / LPI;
  const int sub = threadIdx.x % LPI;
  const int hl = n * D;
  float acc = 0.0f;
  const bool ok = item < T * n;
  const int t = ok ? item / n : 0, hd = ok ? item % n : 0;
  if (ok) {
    const uint4 a = *reinterpret_cast<const uint4*>(dc + t * hl + hd * D + sub * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(c + t * hl + hd * D + sub * 8);
    const uint32_t* wa = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* wb = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += lo_bf(wa[i]) * lo_bf(wb[i]) + hi_bf(wa[i]) * hi_bf(wb[i]);
  }
#pragma unroll
  for (int o = LPI / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (ok && sub == 0) {
    const int bi = t / s, i = t % s;
    delta[(static_cast<size_t>(bi) * n + hd) * s + i] = acc;
  }
}

// ------------------------------------------------------------ dK and dV
// Key rows of 128 (4 waves x 32, lane = key), query stages of QS = 32 staged
// by DMA in a ring of BNST stages (BNST - 1 in flight while one is
// computed), each two row-major tiles, Q (fp16) and dO (A operands of
// S = Q K^T and dP = dO V^T, and, read transposed with the rows in the
// accumulator's order, of dK^T += Q^T dS and dV^T += dO^T P), and the
// stage's log-sum-exp and delta (the same DMA, 32 floats each).
constexpr int QS = 32;
constexpr int BNST = 4;

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const u16* __restrict__ qkv, const u16* __restrict__ qk16, const u16* __restrict__ dcg,
    const float* __restrict__ lse, const float* __restrict__ delta, u16* __restrict__ dz,
    int ld_dz, int s, int n, int window, int nkt, RowSplit rsp) {
  constexpr int NKS = D / 16, ND = D / 32;
  constexpr int OPB = QS * D;  // u16 elements of one operand's tile
  constexpr int STG = 2 * OPB;
  __shared__ __attribute__((aligned(1024))) u16 qs[BNST * STG];
  // per stage: the DMA of the log-sum-exp and of delta, 1 KB each (the first
  // QS floats are the stage's queries; the rest of each KB receives zeros)
  __shared__ __attribute__((aligned(1024))) float ld_lds[BNST][2][256];
  __shared__ int arrival;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const RowBlock rb = row_block(rsp, n);
  const int hd = rb.hd, bi = rb.bi;
  const int hl = n * D, ld = 3 * hl;
  const u16* Qh = qk16 + static_cast<size_t>(bi) * s * (2 * hl) + hd * D;  // fp16
  const u16* Kh = Qh + hl;
  const u16* Vg = qkv + static_cast<size_t>(bi) * s * ld + hd * D + 2 * hl;  // bf16
  const u16* dOg = dcg + static_cast<size_t>(bi) * s * hl + hd * D;
  const float* lse_h = lse + (static_cast<size_t>(bi) * n + hd) * s;
  const float* dl_h = delta + (static_cast<size_t>(bi) * n + hd) * s;
  const RowItem item = decode_row_item<false>(rb.item, nkt, s, window, rsp.ch);
  if (item.nchunks == 0) return;
  const int kb0 = item.row * BKB, kw0 = kb0 + wave * 32, kj = kw0 + l32;

  const int q_begin = item.span.begin;
  const int q_end = item.span.end;
  TileDma<D, QS, false> dq_r, do_r;
  // loads per stage and wave: the two tiles' share, plus the log-sum-exp and
  // delta loads, which every wave issues alike (identical values to the same
  // LDS bytes) so that every wave counts the same loads
  constexpr int LPT = 2 * TileDma<D, QS, false>::LPW + 2;
  dq_r.init(Qh, 2 * hl, s, wave, lane);
  do_r.init(dOg, hl, s, wave, lane);
  const uint32_t qs_lds = __builtin_amdgcn_readfirstlane(lds_address(qs));
  const uint32_t ld_base = __builtin_amdgcn_readfirstlane(lds_address(ld_lds));
  const i32x4 lse_desc = make_desc(reinterpret_cast<const u16*>(lse_h), static_cast<uint32_t>(s) * 4);
  const i32x4 dl_desc = make_desc(reinterpret_cast<const u16*>(dl_h), static_cast<uint32_t>(s) * 4);
  // lanes 0..7 carry the 32 floats of a stage (16 bytes each); the others
  // read out of range (zeros, no memory traffic)
  const int ld_voff = lane < QS / 4 ? lane * 16 : kOutOfRange;
  // stage st <- queries qt0 .. qt0 + QS - 1, or loads that only keep the
  // count in flight constant (qt0 past the span)
  auto issue = [&](int st, int qt0) {
    const uint32_t lds = qs_lds + st * (STG * 2);
    const uint32_t ldl = ld_base + st * (2 * 256 * 4);
    if (qt0 < q_end) {
      dq_r.issue(lds, qt0, wave);
      do_r.issue(lds + OPB * 2, qt0, wave);
      lds_dma16(lse_desc, ldl, ld_voff, qt0 * 4);
      lds_dma16(dl_desc, ldl + 256 * 4, ld_voff, qt0 * 4);
    } else {
      dq_r.issue_none(lds, wave);
      do_r.issue_none(lds + OPB * 2, wave);
      // every lane out of range through its own offset (kOutOfRange + 0
      // cannot wrap below the buffer's size)
      lds_dma16(lse_desc, ldl, kOutOfRange, 0);
      lds_dma16(dl_desc, ldl + 256 * 4, kOutOfRange, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < BNST - 1; ++i) issue(i, q_begin + i * QS);
  // load p of issue alone (p < NP; the same loads, in the same order)
  constexpr int NP = LPT;
  auto issue_piece = [&](int st, int qt0, int p) {
    const uint32_t lds = qs_lds + st * (STG * 2);
    const uint32_t ldl = ld_base + st * (2 * 256 * 4);
    const bool valid = qt0 < q_end;
    constexpr int L = TileDma<D, QS, false>::LPW;
    if (p < L) {
      dq_r.issue_one(lds, qt0, wave, p, valid);
    } else if (p < 2 * L) {
      do_r.issue_one(lds + OPB * 2, qt0, wave, p - L, valid);
    } else if (p == 2 * L) {
      lds_dma16(lse_desc, ldl, valid ? ld_voff : kOutOfRange, valid ? qt0 * 4 : 0);
    } else {
      lds_dma16(dl_desc, ldl + 256 * 4, valid ? ld_voff : kOutOfRange, valid ? qt0 * 4 : 0);
    }
  };

  bf16x8 kf[NKS], vf[NKS];  // fp16 keys, bf16 values of this lane's key
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (kj < s) {
      a = *reinterpret_cast<const uint4*>(Kh + kj * (2 * hl) + ks * 16 + g * 8);
      b = *reinterpret_cast<const uint4*>(Vg + kj * ld + ks * 16 + g * 8);
    }
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(b);
  }
  // The key and value fragments are complete before the loop (the compiler
  // does not see the DMA loads: left to itself it would wait for every
  // outstanding load at their first use inside the loop, every iteration).
  wait_vm_lds<0>();
  const float sc = kLog2e / sqrtf(static_cast<float>(D));
  f32x16 dv[ND], dk[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dv[db][e] = 0.0f; dk[db][e] = 0.0f; }

  int stage = 0;
  for (int qt0 = q_begin; qt0 < q_end; qt0 += QS) {
    // this wave's loads of stage qt0 landed (BNST - 2 later stages' may still
    // be in flight: loads complete in order)
    wait_vm_lds<(BNST - 2) * LPT>();
    __syncthreads();  // every wave's; the stage read last iteration is free again
    const int nst = stage == 0 ? BNST - 1 : stage - 1, nq = qt0 + (BNST - 1) * QS;
    const u16* q_lds = qs + stage * STG;
    const u16* do_lds = q_lds + OPB;
    const float* lse_s = ld_lds[stage][0];
    const float* dl_s = ld_lds[stage][1];

    const bool any = kw0 < s && qt0 + QS - 1 >= kw0 && qt0 - (kw0 + 31) < window;
    if (!any) issue(nst, nq);
    if (any) {
      const bool full = qt0 >= kw0 + 31 && qt0 + QS - 1 - kw0 < window && qt0 + QS <= s;
      // each chain's first product takes a literal zero accumulator (no
      // per-stage zeroing copies of the accumulator registers)
      const f32x16 zero = {};
      f32x16 sp = zero, dp = zero;
      // query fragments of k-step ks + 1 read under the MFMAs of k-step ks
      // (one wave per SIMD: a read issued just before its MFMA would leave
      // the LDS latency exposed)
      bf16x8 fq[2], fdo[2];
      fq[0] = row_frag<D>(q_lds, l32, g);
      fdo[0] = row_frag<D>(do_lds, l32, g);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = ks & 1;
        if (ks + 1 < NKS) {
          fq[c ^ 1] = row_frag<D>(q_lds, l32, (ks + 1) * 2 + g);
          fdo[c ^ 1] = row_frag<D>(do_lds, l32, (ks + 1) * 2 + g);
        }
        if (ks > 0) asm volatile("" : "+v"(fq[c]), "+v"(fdo[c]));
        sp = mfma32x32x16_f16(fq[c], kf[ks], ks == 0 ? zero : sp);
        dp = mfma32x32x16(fdo[c], vf[ks], ks == 0 ? zero : dp);
        // the next stage's loads after the first NP pairs of products, one
        // per pair: with one wave per SIMD, a burst of loads ahead of the
        // products would hold them all up while the loads wait to issue.
        // The empty asm statements (no instructions) keep that order.
        if (ks < NP) {
          asm volatile("" ::"a"(sp), "a"(dp));
          issue_piece(nst, nq, ks);
        }
        if (ks + 1 < NKS) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMAs
        }
      }
      static_assert(NP <= NKS, "one load per pair of products");
      if (!full) {
        // a stage on the diagonal or the window's edge: keep queries in
        // [lo, hi] of this lane's key, as offsets from the lane's first query
        asm volatile("; masked query stage");  // keeps this path a real branch
        const int base = qt0 + g * 4;
        const int lo = kj - base;
        const int hi = min(kj + window - 1, s - 1) - base;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = (e >> 2) * 8 + (e & 3);
          if (off < lo || off > hi) sp[e] = -INFINITY;
        }
      }
      // accumulator element e holds query 8 (e / 4) + 4 g + e % 4
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 lv = *reinterpret_cast<const float4*>(lse_s + 8 * j + 4 * g);
        const float4 dlv = *reinterpret_cast<const float4*>(dl_s + 8 * j + 4 * g);
        const float lq[4] = {lv.x, lv.y, lv.z, lv.w};
        const float dq[4] = {dlv.x, dlv.y, dlv.z, dlv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * j + i;
          const float p = __builtin_amdgcn_exp2f(fmaf(sp[e], sc, -lq[i]));
          sp[e] = p;
          dp[e] = p * (dp[e] - dq[i]);
        }
      }
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const bf16x8 pb = pack8(sp, e2 * 8);
        const bf16x8 dsh = pack8h(dp, e2 * 8);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          dv[db] = mfma32x32x16(frag_rows_tr<D>(do_lds, db * 32, e2, lane), pb, dv[db]);
          dk[db] = mfma32x32x16_f16(frag_rows_tr<D>(q_lds, db * 32, e2, lane), dsh, dk[db]);
        }
      }
    }
    stage = stage == BNST - 1 ? 0 : stage + 1;
  }
  // the trailing loads (beyond the span) land before the LDS can be reused
  wait_vm_lds<0>();

  if (item.nchunks > 1) {
    // A chunk of a split key row: store dk, dv (device scope), count in; the
    // last chunk to arrive sums all of them, in chunk order.
    constexpr int PER_SLOT = 2 * BKB * D;
    const size_t row_id = (static_cast<size_t>(bi) * n + hd) * nkt + item.row;
    const size_t slot0 = (static_cast<size_t>(bi) * n + hd) * rsp.split_slots;
    const int first_slot = item.slot - item.chunk;
    {
      const __amdgpu_buffer_rsrc_t pr = dev_rsrc(rsp.partials + (slot0 + item.slot) * PER_SLOT, PER_SLOT);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        st16_dev(pr, (wave * ND + db) * 1024, lane, dk[db]);
        st16_dev(pr, BKB * D + (wave * ND + db) * 1024, lane, dv[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) arrival = atomicAdd(rsp.counters + row_id, 1);
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(arrival) != item.nchunks - 1) return;
    if (tid == 0) rsp.counters[row_id] = 0;
    // At d = 128 (one workgroup per CU) this chunk's own partial stays in
    // registers and only the others are loaded back; the smaller build would
    // lose its second workgroup per CU to the copy. The sum keeps chunk order.
    constexpr bool OWN = D == 128;
    f32x16 ok[OWN ? ND : 1], ov[OWN ? ND : 1];
    if constexpr (OWN) {
#pragma unroll
      for (int db = 0; db < ND; ++db) { ok[db] = dk[db]; ov[db] = dv[db]; }
    }
    for (int c = 0; c < item.nchunks; ++c) {
      f32x16 a[ND], v[ND];
      if (OWN && c == item.chunk) {
#pragma unroll
        for (int db = 0; db < ND; ++db) { a[db] = ok[OWN ? db : 0]; v[db] = ov[OWN ? db : 0]; }
      } else {
        const __amdgpu_buffer_rsrc_t pr =
            dev_rsrc(rsp.partials + (slot0 + first_slot + c) * PER_SLOT, PER_SLOT);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          ld16_dev(pr, (wave * ND + db) * 1024, lane, reinterpret_cast<float*>(&a[db]));
          ld16_dev(pr, BKB * D + (wave * ND + db) * 1024, lane, reinterpret_cast<float*>(&v[db]));
        }
      }
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          dk[db][e] = c == 0 ? a[db][e] : dk[db][e] + a[db][e];
          dv[db][e] = c == 0 ? v[db][e] : dv[db][e] + v[db][e];
        }
    }
  }

  if (kj < s) {
    const float rs = 1.0f / sqrtf(static_cast<float>(D));
    u16* row = dz + (static_cast<size_t>(bi) * s + kj) * ld_dz + hd * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = db * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2*>(row + hl + d0) =
            make_uint2(pack2bf(dk[db][jj * 4 + 0] * rs, dk[db][jj * 4 + 1] * rs),
                       pack2bf(dk[db][jj * 4 + 2] * rs, dk[db][jj * 4 + 3] * rs));
        *reinterpret_cast<uint2*>(row + 2 * hl + d0) =
            make_uint2(pack2bf(dv[db][jj * 4 + 0], dv[db][jj * 4 + 1]),
                       pack2bf(dv[db][jj * 4 + 2], dv[db][jj * 4 + 3]));
      }
  }
}

// ------------------------------------------------------------------- dQ
// Query rows of 128 (4 waves x 32), key tiles of BKQ staged by DMA in a ring
// of QNST stages (QNST - 1 in flight while one is computed), each two
// row-major tiles: K (fp16) and V (the A operands of S^T = K Q^T and
// dP^T = V dO^T; K read transposed, rows in the accumulator's order, is also
// the A operand of dQ^T += K^T dS^T).  With 32-key tiles a stage takes 16 KB
// for D = 128 and two workgroups share a CU, so one wave's softmax runs under
// the other's MFMAs.
constexpr int BKQ = 32;
constexpr int QNST = 4;
constexpr int KBQ = BKQ / 32;  // 32 x 32 S^T blocks per tile
template <int D>
__global__ __launch_bounds__(256, BKQ == 32 ? 2 : 1) void attn_bwd_dq_kernel(
    const u16* __restrict__ qkv, const u16* __restrict__ qk16, const u16* __restrict__ dcg,
    const float* __restrict__ lse, const float* __restrict__ delta, u16* __restrict__ dz,
    int ld_dz, int s, int n, int window, int nqt, RowSplit rsp) {
  constexpr int NKS = D / 16, ND = D / 32;
  constexpr int OPB = BKQ * D;  // u16 elements of one operand's tile
  constexpr int STG = 2 * OPB;  // one stage: K (fp16), V (bf16)
  __shared__ __attribute__((aligned(1024))) u16 kv[QNST * STG];
  __shared__ int arrival;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const RowBlock rb = row_block(rsp, n);
  const RowItem item = decode_row_item<true>(rb.item, nqt, s, window, rsp.ch);
  if (item.nchunks == 0) return;
  const int qt = item.row;
  const int hd = rb.hd, bi = rb.bi;
  const int hl = n * D, ld = 3 * hl;
  const u16* Qh = qk16 + static_cast<size_t>(bi) * s * (2 * hl) + hd * D;  // fp16
  const u16* Kh = Qh + hl;
  const u16* Vg = qkv + static_cast<size_t>(bi) * s * ld + hd * D + 2 * hl;  // bf16
  const u16* dOg = dcg + static_cast<size_t>(bi) * s * hl + hd * D;
  const int q0 = qt * BQ, qw0 = q0 + wave * 32, qi = qw0 + l32;

  const int kv_begin = item.span.begin;
  const int kv_end = item.span.end;
  TileDma<D, BKQ, false> dk, dv;
  constexpr int LPT = 2 * TileDma<D, BKQ, false>::LPW;  // loads per tile and wave
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
#pragma unroll
  for (int i = 0; i < QNST - 1; ++i) issue(i, kv_begin + i * BKQ);

  bf16x8 qf[NKS], of[NKS];  // fp16 query, bf16 dO fragments of this lane's query
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (qi < s) {
      a = *reinterpret_cast<const uint4*>(Qh + qi * (2 * hl) + ks * 16 + g * 8);
      b = *reinterpret_cast<const uint4*>(dOg + qi * hl + ks * 16 + g * 8);
    }
    qf[ks] = as_bf16x8(a);
    of[ks] = as_bf16x8(b);
  }
  const size_t hrow = (static_cast<size_t>(bi) * n + hd) * s;
  const float lq = qi < s ? lse[hrow + qi] : 0.0f;
  const float dq_delta = qi < s ? delta[hrow + qi] : 0.0f;
  const float sc = kLog2e / sqrtf(static_cast<float>(D));
  // every one of these loads complete before the loop (see the dK/dV kernel)
  wait_vm_lds<0>();

  f32x16 dq[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.0f;

  int stage = 0;
  for (int kt0 = kv_begin; kt0 < kv_end; kt0 += BKQ) {
    // this wave's loads of tile kt0 landed (QNST - 2 later tiles' may still
    // be in flight: loads complete in order)
    wait_vm_lds<(QNST - 2) * LPT>();
    __syncthreads();  // every wave's; the stage read last iteration is free again
    issue(stage == 0 ? QNST - 1 : stage - 1, kt0 + (QNST - 1) * BKQ);
    const u16* k_lds = kv + stage * STG;
    const u16* v_lds = k_lds + OPB;
    stage = stage == QNST - 1 ? 0 : stage + 1;

    const bool any = qw0 < s && qw0 + 31 >= kt0 && qw0 - (kt0 + BKQ - 1) < window;
    if (!any) continue;
    const bool full = kt0 + BKQ - 1 <= qw0 && qw0 + 31 - kt0 < window && kt0 + BKQ <= s;

    // each chain's first product takes a literal zero accumulator
    const f32x16 zero = {};
    f32x16 st[KBQ], dpt[KBQ];
#pragma unroll
    for (int kb = 0; kb < KBQ; ++kb) {
      st[kb] = zero;
      dpt[kb] = zero;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        st[kb] = mfma32x32x16_f16(row_frag<D>(k_lds, kb * 32 + l32, ks * 2 + g), qf[ks],
                                  ks == 0 ? zero : st[kb]);
        dpt[kb] = mfma32x32x16(row_frag<D>(v_lds, kb * 32 + l32, ks * 2 + g), of[ks],
                               ks == 0 ? zero : dpt[kb]);
      }
    }
    if (!full) {
      // a tile on the diagonal or the window's edge: keep keys in [lo, hi]
      // of this lane's query, as offsets from the lane's first key
      asm volatile("; masked key tile");  // keeps this path a real branch
      const int base = kt0 + g * 4;
      const int lo = max(qi - window + 1, 0) - base;
      const int hi = min(qi, s - 1) - base;
#pragma unroll
      for (int kb = 0; kb < KBQ; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kb * 32 + (e >> 2) * 8 + (e & 3);
          if (off < lo || off > hi) st[kb][e] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KBQ; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[kb][e], sc, -lq));
        st[kb][e] = p * (dpt[kb][e] - dq_delta);
      }
#pragma unroll
    for (int kb = 0; kb < KBQ; ++kb)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const bf16x8 dsh = pack8h(st[kb], e2 * 8);
#pragma unroll
        for (int db = 0; db < ND; ++db)
          dq[db] = mfma32x32x16_f16(frag_rows_tr<D>(k_lds, db * 32, kb * 2 + e2, lane), dsh, dq[db]);
      }
  }

  // the trailing loads (beyond the span) land before the LDS can be reused
  wait_vm_lds<0>();

  if (item.nchunks > 1) {
    // A chunk of a split query row: store dq (device scope), count in; the
    // last chunk to arrive sums all of them, in chunk order.
    constexpr int PER_SLOT = BQ * D;
    const size_t row_id = (static_cast<size_t>(bi) * n + hd) * nqt + qt;
    const size_t slot0 = (static_cast<size_t>(bi) * n + hd) * rsp.split_slots;
    const int first_slot = item.slot - item.chunk;
    {
      const __amdgpu_buffer_rsrc_t pr = dev_rsrc(rsp.partials + (slot0 + item.slot) * PER_SLOT, PER_SLOT);
#pragma unroll
      for (int db = 0; db < ND; ++db) st16_dev(pr, (wave * ND + db) * 1024, lane, dq[db]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) arrival = atomicAdd(rsp.counters + row_id, 1);
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(arrival) != item.nchunks - 1) return;
    if (tid == 0) rsp.counters[row_id] = 0;
    // This chunk's own partial is still in registers: only the others are
    // loaded back, and the sum keeps chunk order.
    f32x16 oq[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oq[db] = dq[db];
    for (int c = 0; c < item.nchunks; ++c) {
      f32x16 a[ND];
      if (c == item.chunk) {
#pragma unroll
        for (int db = 0; db < ND; ++db) a[db] = oq[db];
      } else {
        const __amdgpu_buffer_rsrc_t pr =
            dev_rsrc(rsp.partials + (slot0 + first_slot + c) * PER_SLOT, PER_SLOT);
#pragma unroll
        for (int db = 0; db < ND; ++db) ld16_dev(pr, (wave * ND + db) * 1024, lane, reinterpret_cast<float*>(&a[db]));
      }
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[db][e] = c == 0 ? a[db][e] : dq[db][e] + a[db][e];
    }
  }

  if (qi < s) {
    const float rs = 1.0f / sqrtf(static_cast<float>(D));
    u16* row = dz + (static_cast<size_t>(bi) * s + qi) * ld_dz + hd * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = db * 32 + jj * 8 + g * 4;
        *reinterpret_cast<uint2*>(row + d0) =
            make_uint2(pack2bf(dq[db][jj * 4 + 0] * rs, dq[db][jj * 4 + 1] * rs),
                       pack2bf(dq[db][jj * 4 + 2] * rs, dq[db][jj * 4 + 3] * rs));
      }
  }
}

template <int D>
hipError_t bwd_d(const u16* qkv, const u16* qk16, const u16* c, const float* lse,
                 const u16* dc, float* delta, u16* dz, int ld_dz, int b, int s, int n,
                 int window, const AttnScratch& sc, hipStream_t st) {
  const int T = b * s;
  const long items = static_cast<long>(T) * n;
  const int per_block = 256 / (D / 8);
  hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((items + per_block - 1) / per_block), dim3(256),
                     0, st, dc, c, delta, T, s, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkt = (s + BKB - 1) / BKB;
  RowSplit rk;
  int kitems = 0;
  e = plan_rows<false>(b, s, n, window, nkt, 2 * BKB * D, launch_slots(attn_bwd_dkdv_kernel<D>, sc),
                       sc, &rk, &kitems);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3(kitems * rk.nb), dim3(256), 0, st, qkv, qk16,
                     dc, lse, delta, dz, ld_dz, s, n, window, nkt, rk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqt = (s + BQ - 1) / BQ;
  RowSplit rq;
  int qitems = 0;
  e = plan_rows<true>(b, s, n, window, nqt, BQ * D, launch_slots(attn_bwd_dq_kernel<D>, sc), sc,
                      &rq, &qitems);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(qitems * rq.nb), dim3(256), 0, st, qkv, qk16, dc,
                     lse, delta, dz, ld_dz, s, n, window, nqt, rq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd(const u16* qkv, const u16* qk16, const u16* c,
                                const float* lse, const u16* dc, float* delta, u16* dz,
                                int ld_dz, int b, int s, int n, int d, int window,
                                const AttnScratch& sc, hipStream_t st) {
  if (d == 128)
    return bwd_d<128>(qkv, qk16, c, lse, dc, delta, dz, ld_dz, b, s, n, window, sc, st);
  if (d == 64)
    return bwd_d<64>(qkv, qk16, c, lse, dc, delta, dz, ld_dz, b, s, n, window, sc, st);
  return hipErrorInvalidValue;
}

}  // namespace ptb
