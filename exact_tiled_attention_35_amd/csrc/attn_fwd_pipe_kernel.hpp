// Exact tiled attention forward for head dimension 256, software-pipelined
// inside each wave (gfx950).
//
// Same computation and tiling as attn_fwd_kernel (softmax(Q K^T * scale) V
// per (batch, query head), the formula of the interface section of
// hysenlabs.com's "FlashAttention: exakte Attention-Kernel fuer CUDA und
// ROCm"; stages 1-4 of the five-stage map in unite.ai's "Was ist
// FlashAttention?", section "Eine fuenfstufige Betriebsuebersicht"), laid out
// differently for stage 5, the target accelerator:
//
//  * At d = 256 the 128 O^T accumulators of a wave's 32 query rows leave room
//    for one wave per SIMD only, so no second wave fills the issue slots while
//    a wave waits on its own matrix results: with one tile in flight the
//    softmax and the MFMAs run back to back (counters: 9 of 1,022 MFMA-busy
//    cycles per tile co-issue a VALU instruction).
//  * Here each wave computes S^T of tile t+1 while it exponentiates tile t:
//    the 32 MFMAs of the next S^T product and the exp2 / sum of the current
//    tile sit in one basic block, interleaved two MFMAs to a few VALU
//    instructions, so that the VALU work issues in the shadow of the matrix
//    work.  Then O^T += V^T P^T for tile t.
//  * The products run on v_mfma_f32_16x16x32 in the layout of
//    attn_fwd_k16_kernel (lane group g = l / 16 and c = l % 16: S^T and O^T
//    in 16 x 16 blocks, two query blocks per wave, P^T packed from the S^T
//    registers, V^T from two transpose reads per operand; K, Q and V rows
//    padded to 8 (mod 16) dwords, free of LDS bank conflicts): 1.2-2.7 %
//    faster than the same pipeline on v_mfma_f32_32x32x16.
//  * K therefore runs one tile ahead of V: three K stages (tile t for the
//    rare recomputation of a lean tile, t+1 being multiplied, t+2 loading)
//    and two V stages (t being multiplied, t+1 loading), plus the LDS copy of
//    the workgroup's Q tile: 153 KB of the 160 KB LDS.  One barrier per tile,
//    as in attn_fwd_kernel.
//
// Plain instances only (no score variants, packed sequences or block mask);
// scale > 0 (the launcher sends other scales to attn_fwd_kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd_kernel.hpp"
#include "gfx950_ops.hpp"

namespace eta {

template <int D>
struct PipeCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;  // query rows per workgroup
  static constexpr int BN = 32;           // keys per K/V tile
  static constexpr int kChunks = D / 8;   // 16-byte chunks per row
  static constexpr int KCP = kChunks + 2; // K (and Q) row, in 16-byte slots
  static constexpr int VCP = kChunks + 2; // V row, in 16-byte slots
  static constexpr int KS = 8 * KCP;      // K / Q row stride (elements)
  static constexpr int VS = 8 * VCP;      // V row stride (elements)
  static constexpr int kKInst = (BN * KCP + 63) / 64;
  static constexpr int kVInst = (BN * VCP + 63) / 64;
  static constexpr int kQInst = (BM * KCP + 63) / 64;
  static constexpr int kKElems = kKInst * 64 * 8;
  static constexpr int kVElems = kVInst * 64 * 8;
  static constexpr int kQElems = kQInst * 64 * 8;
  static constexpr int kKStages = 3, kVStages = 2;
  static constexpr int kVBase = kKStages * kKElems;
  static constexpr int kQBase = kVBase + kVStages * kVElems;
  static constexpr int kLdsElems = kQBase + kQElems;
  static constexpr int kKInstPerWave = (kKInst + kWaves - 1) / kWaves;
  static constexpr int kVInstPerWave = (kVInst + kWaves - 1) / kWaves;
  static constexpr int kQInstPerWave = (kQInst + kWaves - 1) / kWaves;
  static_assert(D == 256, "the pipelined kernel is laid out for d = 256");
  static_assert((KS / 2) % 16 == 8 && (VS / 2) % 16 == 8, "conflict-free row strides");
  static_assert(kLdsElems * 2 <= 160 * 1024, "LDS of one workgroup");
  static_assert(kWaves * 32 * (D + 8) <= kLdsElems, "the epilogue's staged rows fit");
};

template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(PipeCfg<D>::kThreads, 1)
attn_fwd_pipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb, int total,
                     float c_log2) {
  using C = PipeCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NK4 = D / 32;  // 32-wide k-steps of S^T
  constexpr int NDB = D / 16;  // 16-dimension blocks of O^T
  static_assert(BN == 32, "one 32-key step of the PV product per tile");

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;

  const WorkItem w = map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int diag = Nk - Nq;  // causal: key j visible to row i iff j <= i + diag

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const int64_t qo_off = ((int64_t)w.b * Nq + qw0) * q_rs + (int64_t)w.hq * D;
  const uint16_t* Kh = K + ((int64_t)w.b * Nk * Hkv + hkv) * D;
  const uint16_t* Vh = V + ((int64_t)w.b * Nk * Hkv + hkv) * D;
  const int64_t lse_off = ((int64_t)w.b * Hq + w.hq) * Nq;

  // ---- The workgroup's Q tile into LDS (rows past Nq read as zero).
  uint16_t* const qs = smem + C::kQBase;
  {
    const int64_t q0_off = ((int64_t)w.b * Nq + q0) * q_rs + (int64_t)w.hq * D;
    const rsrc_t qr = make_rsrc(Q + q0_off, span_bytes(q0, BM, Nq, q_rs, D));
#pragma unroll
    for (int i = 0; i < C::kQInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      const int sl = 64 * j + lane;
      const int row = min(sl / C::KCP, BM - 1), ch = min(sl % C::KCP, C::kChunks - 1);
      if (j < C::kQInst) buf_load_lds16(qr, qs + 512 * j, (int)(row * q_rs * 2) + 16 * ch);
    }
  }

  // ---- Key range of the workgroup (nt tiles) and of this wave (wt tiles:
  // a wave computes tiles 0 .. wt-1 and only takes part in the loads and
  // barriers of the rest).  Tiles before nf are visible to every row.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);
  const int wt = w_end > 0 ? min(nt, (w_end + BN - 1) / BN) : 0;
  int nf = Nk / BN;
  if (CAUSAL) nf = min(nf, max(0, (q0 + diag + 1) / BN));
  nf = min(max(nf, 0), nt);

  // ---- Direct global->LDS tile loads (loop-invariant per-lane offsets).
  int koff[C::kKInstPerWave], voff[C::kVInstPerWave];
#pragma unroll
  for (int i = 0; i < C::kKInstPerWave; ++i) {
    const int sl = 64 * (wave + C::kWaves * i) + lane;
    const int row = min(sl / C::KCP, BN - 1), ch = min(sl % C::KCP, C::kChunks - 1);
    koff[i] = (int)(row * kv_rs * 2) + 16 * ch;
  }
#pragma unroll
  for (int i = 0; i < C::kVInstPerWave; ++i) {
    const int sl = 64 * (wave + C::kWaves * i) + lane;
    const int row = min(sl / C::VCP, BN - 1), ch = min(sl % C::VCP, C::kChunks - 1);
    voff[i] = (int)(row * kv_rs * 2) + 16 * ch;
  }
  auto issue_k = [&](int t, uint16_t* __restrict__ st) {
    const int j0 = t * BN;
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, span_bytes(j0, BN, Nk, kv_rs, D));
#pragma unroll
    for (int i = 0; i < C::kKInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      if (j < C::kKInst) buf_load_lds16(kr, st + 512 * j, koff[i]);
    }
  };
  auto issue_v = [&](int t, uint16_t* __restrict__ st) {
    const int j0 = t * BN;
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, span_bytes(j0, BN, Nk, kv_rs, D));
#pragma unroll
    for (int i = 0; i < C::kVInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      if (j < C::kVInst) buf_load_lds16(vr, st + 512 * j, voff[i]);
    }
  };
  auto kstage = [&](int t) { return smem + (t % C::kKStages) * C::kKElems; };
  auto vstage = [&](int t) { return smem + C::kVBase + (t & 1) * C::kVElems; };

  // ---- Operand reads from LDS (16x16x32 layout; lane group g = l / 16,
  // c = l % 16): K row 16 kb + c and Q row 16 qb + c of this wave, columns
  // 32 k4 + 8 g; for the V transpose reads lane c of group g addresses row
  // 4 g + c / 4 (+ 16 for the second half of the key step) at column
  // 4 (c % 4) of the 16-column block.
  const int k_rd = c * KS + 8 * g;
  const int q_rd = C::kQBase + (wave * 32 + c) * KS + 8 * g;
  const int v_rd = (4 * g + (c >> 2)) * VS + 4 * (c & 3);
  auto rd16 = [](const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); };

  // O^T in 16 x 16 blocks: oacc[qb][db] register r holds dimension
  // 16 db + 4 g + r of query qw0 + 16 qb + c.
  f32x4_t oacc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x4_t{};
  float m[2] = {-INFINITY, -INFINITY};  // running max of s * c_log2 (log2 units)
  float lsum[2] = {0.f, 0.f};           // this lane's share of the running sums

  // S^T (32 keys x 32 queries) from the K stage at kst in 16 x 16 blocks
  // s[qb][kb] (register r: key 16 kb + 4 g + r, query 16 qb + c); per
  // k-step each K operand feeds two consecutive MFMAs (measured 1.5 %
  // faster here than sharing the Q^T operand instead).
  using SBlk = f32x4_t[2][2];
  auto compute_s = [&](const uint16_t* kst, SBlk& s) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x4_t{};
#pragma unroll
    for (int k4 = 0; k4 < NK4; ++k4) {
      const u32x4_t b0 = rd16(smem + q_rd + 32 * k4), b1 = rd16(smem + q_rd + 16 * KS + 32 * k4);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t a = rd16(kst + k_rd + kb * 16 * KS + 32 * k4);
        s[0][kb] = mfma_16x16x32<BF16>(a, b0, s[0][kb]);
        s[1][kb] = mfma_16x16x32<BF16>(a, b1, s[1][kb]);
      }
    }
  };

  // Row maximum of block qb over the tile (in-lane, then across the four
  // lane groups); m is raised when the tile max exceeds it by more than
  // `threshold`, and what was accumulated is rescaled.
  auto raise_max = [&](int qb, const f32x4_t (&s)[2], float threshold) {
    float tmax = max3(max3(s[0][0], s[0][1], s[0][2]), s[0][3], s[1][0]);
    tmax = max3(tmax, max3(s[1][1], s[1][2], s[1][3]), tmax);
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
    const float tm = tmax * c_log2;
    if (tm > m[qb] + threshold) {
      const float alpha = exp2_fast(m[qb] - tm);
      m[qb] = tm;
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
    }
  };

  // p = 2^(s*c - m) in place for block qb; returns this lane's sum of the
  // unrounded p.
  auto exponentiate = [&](int qb, f32x4_t (&s)[2]) {
    const float mb = m[qb] != -INFINITY ? m[qb] : 0.f;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(s[kb][r], c_log2, -mb));
        const float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], c_log2, -mb));
        s[kb][r] = p0;
        s[kb][r + 1] = p1;
        ps0 += p0;
        ps1 += p1;
      }
    }
    return ps0 + ps1;
  };

  // O^T += V^T P^T from the V stage at vst: lane group g feeds the keys
  // {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}, the registers of S^T blocks
  // kb = 0 and 1; P as hi + lo on masked causal tiles.  Each V^T operand
  // feeds two consecutive MFMAs (the two query blocks).
  auto pv = [&](const uint16_t* vst, const SBlk& p, auto with_lo) {
    u32x4_t phi[2], plo[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x8_t pv8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv8[e] = p[qb][0][e];
        pv8[4 + e] = p[qb][1][e];
      }
      phi[qb] = pack8<BF16>(pv8);
      if constexpr (decltype(with_lo)::value) plo[qb] = pack8<BF16>(pv8 - unpack8<BF16>(phi[qb]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2_t x0 = lds_read_tr4(vst + v_rd + 16 * db);
      const u32x2_t x1 = lds_read_tr4(vst + v_rd + 16 * VS + 16 * db);
      const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        oacc[qb][db] = mfma_16x16x32<BF16>(a, phi[qb], oacc[qb][db]);
        if constexpr (decltype(with_lo)::value) oacc[qb][db] = mfma_16x16x32<BF16>(a, plo[qb], oacc[qb][db]);
      }
    }
  };

  // Iteration t: K of tile t+2 and V of tile t+1 stream into the stages kl
  // and vl while this wave computes its tile t from the stages kc (K of t),
  // kn (K of t+1) and vc (V of t); the barrier at the end follows the wait
  // for this wave's loads.  The stages arrive as restrict-qualified
  // parameters: the transpose reads of vc then carry alias information that
  // sets them apart from the direct-to-LDS loads just issued, and need not
  // wait for them.
  //
  // kLeanNext: a lean tile (every key visible to every row, m finite) whose
  // successor this wave also computes.  The 16 exponentials of s_cur are
  // interleaved with the 32 S^T MFMAs of tile t+1 into s_next, one score per
  // two MFMAs (the two that share a K operand), each step fenced so that the
  // scheduler keeps the interleave; the K and Q operand reads run two
  // k-steps ahead.  A partial row sum
  // above kSumLimit (a score far above m, rare) recomputes S of tile t from
  // kc and takes the maximum path.
  // kOther: any other tile of this wave (the first, the masked ones, a lean
  // tile without a successor): the maximum path with masking where the tile
  // crosses the causal diagonal or the ragged end, then S^T of tile t+1 if
  // this wave computes it.
  constexpr int kLeanNext = 0, kOther = 1;
  auto step = [&](int t, auto kind, SBlk& s_cur, SBlk& s_next,
                  uint16_t* __restrict__ kl, uint16_t* __restrict__ vl,
                  const uint16_t* __restrict__ kc, const uint16_t* __restrict__ kn,
                  const uint16_t* __restrict__ vc) {
    if (t + 2 < nt) issue_k(t + 2, kl);
    if (t + 1 < nt) issue_v(t + 1, vl);
    if constexpr (decltype(kind)::value == kLeanNext) {
      float ps[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
      SBlk sn;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sn[qb][kb] = f32x4_t{};
      // operands of k-step k4: ka[k4 % 3][kb], qa[k4 % 3][qb]
      u32x4_t ka[3][2], qa[3][2];
      auto fetch = [&](int k4) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          ka[k4 % 3][x] = rd16(kn + k_rd + x * 16 * KS + 32 * k4);
          qa[k4 % 3][x] = rd16(smem + q_rd + x * 16 * KS + 32 * k4);
        }
      };
      fetch(0);
      fetch(1);
#pragma unroll
      for (int k4 = 0; k4 < NK4; ++k4) {
        if (k4 + 2 < NK4) fetch(k4 + 2);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            sn[qb][kb] = mfma_16x16x32<BF16>(ka[k4 % 3][kb], qa[k4 % 3][qb], sn[qb][kb]);
            if (qb == 1) {
              // score i = 2 k4 + kb of the 16: block i / 8, kb (i / 4) % 2, r i % 4
              const int i = 2 * k4 + kb;
              const int eq = i / 8, ekb = (i / 4) % 2, er = i % 4;
              const float p = exp2_fast(__builtin_fmaf(s_cur[eq][ekb][er], c_log2, -m[eq]));
              s_cur[eq][ekb][er] = p;
              ps[eq][er & 1] += p;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_next[qb][kb] = sn[qb][kb];
      float psum[2];
      bool over = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        psum[qb] = ps[qb][0] + ps[qb][1];
        over = over || !(psum[qb] <= kSumLimit);
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        compute_s(kc, s_cur);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          raise_max(qb, s_cur[qb], 0.0f);
          psum[qb] = exponentiate(qb, s_cur[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) lsum[qb] += psum[qb];
      pv(vc, s_cur, std::false_type{});
    } else if (t < wt) {
      const int j0 = t * BN;
      const bool lean = t >= 1 && t < nf;
      bool need_mask = false;
      if (lean) {
        float psum[2];
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          psum[qb] = exponentiate(qb, s_cur[qb]);
          over = over || !(psum[qb] <= kSumLimit);
        }
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
          compute_s(kc, s_cur);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            raise_max(qb, s_cur[qb], 0.0f);
            psum[qb] = exponentiate(qb, s_cur[qb]);
          }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) lsum[qb] += psum[qb];
      } else {
        need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (need_mask) {
            const int my_q = qw0 + 16 * qb + c;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = j0 + 16 * kb + 4 * g + r;
                const bool vis = j < Nk && (!CAUSAL || j <= my_q + diag);
                s_cur[qb][kb][r] = vis ? s_cur[qb][kb][r] : -INFINITY;
              }
            }
          }
          raise_max(qb, s_cur[qb], kRescaleThreshold);
          lsum[qb] += exponentiate(qb, s_cur[qb]);
        }
      }
      if (t + 1 < wt) compute_s(kn, s_next);
      if (CAUSAL && need_mask)
        pv(vc, s_cur, std::true_type{});
      else
        pv(vc, s_cur, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  using LeanNext = std::integral_constant<int, kLeanNext>;
  using Other = std::integral_constant<int, kOther>;
  auto run = [&](int t, auto kind, SBlk& s_cur, SBlk& s_next) {
    step(t, kind, s_cur, s_next, kstage(t + 2), vstage(t + 1), kstage(t), kstage(t + 1),
         vstage(t));
  };
  auto copy_s = [](SBlk& dst, const SBlk& src) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dst[qb][kb] = src[qb][kb];
  };

  // ---- Prologue: Q, K tiles 0 and 1, V tile 0; S of tile 0.
  if (nt > 0) {
    issue_k(0, kstage(0));
    issue_v(0, vstage(0));
  }
  if (nt > 1) issue_k(1, kstage(1));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  SBlk sa, sb;
  if (wt > 0) compute_s(kstage(0), sa);

  // Tile 0 (m = -inf: maximum path), then the lean tiles with a successor
  // two per trip (the roles of sa and sb alternate), then the rest.
  int t = 0;
  if (nt > 0) {
    run(0, Other{}, sa, sb);
    t = 1;
  }
  const int lean_end = max(t, min(nf, wt - 1));  // lean tiles [1, lean_end) have a successor
  for (; t + 1 < lean_end; t += 2) {
    run(t, LeanNext{}, sb, sa);
    run(t + 1, LeanNext{}, sa, sb);
  }
  if (t < lean_end) {
    run(t, LeanNext{}, sb, sa);
    copy_s(sb, sa);
    ++t;
  }
  for (; t < nt; ++t) {
    run(t, Other{}, sb, sa);
    copy_s(sb, sa);
  }

  // ---- Epilogue (every wave passed the last barrier: the stages are idle).
  // Rows are normalised, rounded and staged in this wave's slice of LDS (row
  // 16 qb + c, 4 dimensions per block and lane group), then stored 16
  // contiguous bytes per lane.
  constexpr int ORS = D + 8;
  uint16_t* const ost = smem + wave * 32 * ORS;
  float lt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    lt[qb] = l;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<u32x2_t*>(ost + (16 * qb + c) * ORS + 16 * db + 4 * g) =
          pack4<BF16>(oacc[qb][db] * inv);
  }
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int rr = lane / CPR, cc = lane % CPR;
  const rsrc_t orr = make_rsrc(O + qo_off, span_bytes(qw0, 32, Nq, q_rs, D));
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + rr;
    buf_store16(*reinterpret_cast<const u32x4_t*>(ost + row * ORS + 8 * cc), orr,
                (int)(row * q_rs * 2) + 16 * cc);
  }
  const int nrows = max(0, min(32, Nq - qw0));
  const rsrc_t lr = make_rsrc(LSE + lse_off + qw0, nrows * 4);
  if (g == 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      buf_store4(lt[qb] > 0.f ? (m[qb] + __builtin_amdgcn_logf(lt[qb])) * kLn2 : -INFINITY, lr,
                 4 * (16 * qb + c));
  }
}

}  // namespace eta
