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
//    the 16 MFMAs of the next S^T product and the exp2 / sum of the current
//    tile sit in one basic block, interleaved one MFMA to a few VALU
//    instructions, so that the VALU work issues in the shadow of the matrix
//    work.  Then O^T += V^T P^T for tile t.
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
  static constexpr int KCP = kChunks + 1; // K (and Q) row, in 16-byte slots
  static constexpr int VCP = kChunks + 4; // V row, in 16-byte slots
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
  static_assert((KS / 2) % 8 == 4 && (VS / 2) % 32 == 16, "bank-conflict-free strides");
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
  constexpr int NKS = D / 16;  // k-steps of the S^T product
  constexpr int NDB = D / 32;  // 32-column blocks of O^T
  constexpr int NKK = BN / 16; // 16-key steps of the PV product

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const WorkItem w = map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
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
      const int row = min(sl / C::KCP, BM - 1), c = min(sl % C::KCP, C::kChunks - 1);
      if (j < C::kQInst) buf_load_lds16(qr, qs + 512 * j, (int)(row * q_rs * 2) + 16 * c);
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
    const int row = min(sl / C::KCP, BN - 1), c = min(sl % C::KCP, C::kChunks - 1);
    koff[i] = (int)(row * kv_rs * 2) + 16 * c;
  }
#pragma unroll
  for (int i = 0; i < C::kVInstPerWave; ++i) {
    const int sl = 64 * (wave + C::kWaves * i) + lane;
    const int row = min(sl / C::VCP, BN - 1), c = min(sl % C::VCP, C::kChunks - 1);
    voff[i] = (int)(row * kv_rs * 2) + 16 * c;
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

  // ---- Operand reads from LDS.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int k_rd = l32 * KS + 8 * hh;
  const int q_rd = C::kQBase + (wave * 32 + l32) * KS + 8 * hh;
  const int v_rd = (4 * hh + (i16 >> 2)) * VS + 16 * (g16 & 1) + 4 * (i16 & 3);
  auto rd16 = [](const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY;  // running max of t = s * c_log2 (log2 units)
  float lsum = 0.f;     // this lane half's share of the running sum

  // S^T = K Q^T (32 keys x 32 queries) from the K stage at kst.
  auto compute_s = [&](const uint16_t* kst, f32x16_t& s) {
    s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      s = mfma_32x32x16<BF16>(rd16(kst + k_rd + 16 * ks), rd16(smem + q_rd + 16 * ks), s);
  };

  // Tile row maximum; m is raised when the tile max exceeds it by more than
  // `threshold`, and what was accumulated is rescaled.
  auto raise_max = [&](const f32x16_t& s, float threshold) {
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) tmax = max3(tmax, s[r], s[r + 1]);
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
    const float tm = tmax * c_log2;
    if (tm > m + threshold) {
      const float alpha = exp2_fast(m - tm);
      m = tm;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
  };

  // p = 2^(s*c - m) in place; returns this lane half's sum of the unrounded p.
  auto exponentiate = [&](f32x16_t& s) {
    const float mb = m != -INFINITY ? m : 0.f;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(s[r], c_log2, -mb));
      const float p1 = exp2_fast(__builtin_fmaf(s[r + 1], c_log2, -mb));
      s[r] = p0;
      s[r + 1] = p1;
      ps0 += p0;
      ps1 += p1;
    }
    return ps0 + ps1;
  };

  // O^T += V^T P^T from the V stage at vst; P as hi + lo on masked causal
  // tiles.  The V^T operand reads run four MFMAs ahead.
  auto pv = [&](const uint16_t* vst, const f32x16_t& p, auto with_lo) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      f32x8_t pv8;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv8[e] = p[8 * kk + e];
      const u32x4_t phi = pack8<BF16>(pv8);
      u32x4_t plo;
      if constexpr (decltype(with_lo)::value) plo = pack8<BF16>(pv8 - unpack8<BF16>(phi));
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x2_t x0 = lds_read_tr4(vst + v_rd + 16 * kk * VS + 32 * db);
        const u32x2_t x1 = lds_read_tr4(vst + v_rd + (16 * kk + 8) * VS + 32 * db);
        const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
        oacc[db] = mfma_32x32x16<BF16>(a, phi, oacc[db]);
        if constexpr (decltype(with_lo)::value) oacc[db] = mfma_32x32x16<BF16>(a, plo, oacc[db]);
      }
    }
    if constexpr (!decltype(with_lo)::value) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < NKK * NDB - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // Iteration t: K of tile t+2 and V of tile t+1 stream into the stages kl
  // and vl while this wave computes its tile t from the stages kc (K of t),
  // kn (K of t+1) and vc (V of t); the barrier at the end follows the wait
  // for this wave's loads.  The stages arrive as restrict-qualified
  // parameters: the transpose reads of vc then carry alias information that
  // sets them apart from the direct-to-LDS loads just issued, and need not
  // wait for them (without it the compiler waits for every outstanding
  // direct-to-LDS load before a transpose read, and the load latency lands
  // in every iteration).
  //
  // kLeanNext: a lean tile (every key visible to every row, m finite) whose
  // successor this wave also computes.  The exponentials of s_cur are
  // interleaved with the S^T MFMAs of tile t+1 into s_next, one score per
  // MFMA, each step fenced so that the scheduler keeps the interleave; the K
  // and Q operand reads run three steps ahead.  A partial row sum above
  // kSumLimit (a score far above m, rare) recomputes S of tile t from kc and
  // takes the maximum path.
  // kOther: any other tile of this wave (the first, the masked ones, a lean
  // tile without a successor): the maximum path with masking where the tile
  // crosses the causal diagonal or the ragged end, then S^T of tile t+1 if
  // this wave computes it.
  constexpr int kLeanNext = 0, kOther = 1;
  auto step = [&](int t, auto kind, f32x16_t& s_cur, f32x16_t& s_next,
                  uint16_t* __restrict__ kl, uint16_t* __restrict__ vl,
                  const uint16_t* __restrict__ kc, const uint16_t* __restrict__ kn,
                  const uint16_t* __restrict__ vc) {
    if (t + 2 < nt) issue_k(t + 2, kl);
    if (t + 1 < nt) issue_v(t + 1, vl);
    if constexpr (decltype(kind)::value == kLeanNext) {
      const float mb = m;
      float ps0 = 0.f, ps1 = 0.f;
      f32x16_t sn = f32x16_t{};
      u32x4_t ka[4], qa[4];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        ka[i] = rd16(kn + k_rd + 16 * i);
        qa[i] = rd16(smem + q_rd + 16 * i);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 3 < NKS) {
          ka[(ks + 3) & 3] = rd16(kn + k_rd + 16 * (ks + 3));
          qa[(ks + 3) & 3] = rd16(smem + q_rd + 16 * (ks + 3));
        }
        sn = mfma_32x32x16<BF16>(ka[ks & 3], qa[ks & 3], sn);
        const float p = exp2_fast(__builtin_fmaf(s_cur[ks], c_log2, -mb));
        s_cur[ks] = p;
        if (ks & 1)
          ps1 += p;
        else
          ps0 += p;
        __builtin_amdgcn_sched_barrier(0);
      }
      s_next = sn;
      float psum = ps0 + ps1;
      if (__builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) != 0) {
        compute_s(kc, s_cur);
        raise_max(s_cur, 0.0f);
        psum = exponentiate(s_cur);
      }
      lsum += psum;
      pv(vc, s_cur, std::false_type{});
    } else if (t < wt) {
      const int j0 = t * BN;
      const bool lean = t >= 1 && t < nf;
      bool need_mask = false;
      float psum;
      if (lean) {
        psum = exponentiate(s_cur);
        if (__builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) != 0) {
          compute_s(kc, s_cur);
          raise_max(s_cur, 0.0f);
          psum = exponentiate(s_cur);
        }
      } else {
        need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag);
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = j < Nk && (!CAUSAL || j <= my_q + diag);
            s_cur[r] = vis ? s_cur[r] : -INFINITY;
          }
        }
        raise_max(s_cur, kRescaleThreshold);
        psum = exponentiate(s_cur);
      }
      lsum += psum;
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
  auto run = [&](int t, auto kind, f32x16_t& s_cur, f32x16_t& s_next) {
    step(t, kind, s_cur, s_next, kstage(t + 2), vstage(t + 1), kstage(t), kstage(t + 1),
         vstage(t));
  };

  // ---- Prologue: Q, K tiles 0 and 1, V tile 0; S of tile 0.
  if (nt > 0) {
    issue_k(0, kstage(0));
    issue_v(0, vstage(0));
  }
  if (nt > 1) issue_k(1, kstage(1));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16_t sa, sb;
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
    sb = sa;
    ++t;
  }
  for (; t < nt; ++t) {
    run(t, Other{}, sb, sa);
    sb = sa;
  }

  // ---- Epilogue (every wave passed the last barrier: the stages are idle).
  const float lt = lsum + __shfl_xor(lsum, 32);
  store_rows<D, BF16>(smem, wave, lane, oacc, lt > 0.f ? 1.0f / lt : 0.f,
                      make_rsrc(O + qo_off, span_bytes(qw0, 32, Nq, q_rs, D)), q_rs);
  const int nrows = max(0, min(32, Nq - qw0));
  const rsrc_t lr = make_rsrc(LSE + lse_off + qw0, nrows * 4);
  buf_store4(lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY, lr, 4 * l32);
}

}  // namespace eta
