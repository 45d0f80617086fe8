// Exact tiled attention forward on 16x16x32 matrix instructions (gfx950),
// head dimension 64, 128 or 256.
//
// Same computation and pipeline as attn_fwd_kernel (softmax(Q K^T * scale) V
// per (batch, query head), the formula of the interface section of
// hysenlabs.com's "FlashAttention: exakte Attention-Kernel fuer CUDA und
// ROCm"; 32 query rows per wave, K/V tiles in two LDS stages, lazy
// rescaling, lean tiles), with the products on v_mfma_f32_16x16x32 instead
// of v_mfma_f32_32x32x16: the same flops in twice as many instructions of
// half the size, which the matrix cores of this part run at a higher rate
// for the same power.  Two shapes of workgroup:
//  * 4 waves (128 query rows), 64-key tiles, two workgroups per CU: the
//    causal and block-mask instances (a causal workgroup of 256 rows would
//    idle more waves on the diagonal tiles; a mask block is 128 rows);
//  * WIDE: 8 waves (256 query rows), 128-key tiles, one workgroup per CU
//    (147 KB of LDS): the non-causal batched and packed-sequence instances.
//    Each K/V tile is fetched from L2 once for twice as many rows, and a
//    workgroup meets a barrier once per 128 keys instead of 64.  Without a
//    causal mask a wave's work does not depend on the workgroup's other
//    rows, so both instances compute a sequence's rows bit for bit alike.
//  * d = 256: 4 waves, 32-key tiles (two stages of 68 KB), two workgroups
//    per CU.  With 128 O^T and 64 Q^T registers per wave the tile body fits
//    the 256 registers two workgroups leave it only if a diagonal tile's P
//    goes through the matrix cores as a hi sweep over all of V^T followed
//    by a lo sweep (V^T read from LDS twice on those tiles); interleaving
//    the two halves per V^T block spilled 114 registers.
//
// Layout (lane l, g = l / 16, c = l % 16):
//  * S^T = K Q^T in 16 x 16 blocks s[qb][kb]: register r holds key
//    16 kb + 4 g + r against query 16 qb + c.  Each lane owns two query rows
//    (blocks qb = 0, 1), and the four lanes c, c + 16, c + 32, c + 48 share
//    them: a row maximum or sum is an in-lane reduction plus two exchanges.
//    A operand: K row 16 kb + c, columns 32 k4 + 8 g .. + 7 (one 16-byte LDS
//    read); B operand: Q^T, resident in VGPRs.
//  * O^T = V^T P^T in 16 x 16 blocks o[qb][db]: register r holds dimension
//    16 db + 4 g + r of query 16 qb + c.  A 32-key step kk feeds lane group
//    g the keys 32 kk + {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3} -- exactly
//    the registers of S^T blocks 2 kk and 2 kk + 1 -- so P^T packs from the
//    accumulators without exchanges, and the A operand V^T takes the same
//    key order from two LDS transpose reads (4 consecutive keys each).
//  * K and V rows are padded to a stride of 8 (mod 16) dwords, which keeps
//    both operand reads free of LDS bank conflicts (measured).
//
// Plain, packed-sequence (VARLEN) and block-mask (SPARSE) instances, with
// attn_fwd_kernel's work mapping, row offsets and tile walk for the latter
// two: a packed sequence computes bit for bit what the batched instance
// computes on the same rows, and an all-ones block mask what the causal
// batched instance computes (the non-causal batched call walks 128-key
// tiles, the block-mask instance 64-key ones).  Of the score variants only
// the sliding window (WIN, 128-row workgroups; attn_fwd_kernel's key range,
// tile modes and edge masking); scale > 0.  The launcher uses the kernel at
// d = 128, for plain batched calls at d = 256, and for causal calls (batched,
// packed, block mask) at d = 64.  The tile lambdas are forced inline: the window instances, with
// a third tile loop, were otherwise left as calls with the accumulators in
// scratch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd_kernel.hpp"
#include "gfx950_ops.hpp"

namespace eta {

// WIDE: 8 waves (256 query rows) per workgroup and 128-key tiles, one
// workgroup per CU; otherwise 4 waves (128 rows) and 64-key tiles, two
// workgroups per CU.
template <int D, bool WIDE = false>
struct K16Cfg {
  static constexpr int kWaves = WIDE ? 8 : 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;                 // query rows per workgroup
  static constexpr int BN = WIDE ? 128 : (D == 256 ? 32 : 64);  // keys per K/V tile
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int KCP = kChunks + 2;                // K row, in 16-byte slots
  static constexpr int VCP = kChunks + 2;                // V row, in 16-byte slots
  static constexpr int KS = 8 * KCP, VS = 8 * VCP;       // row strides (elements)
  static constexpr int kKInst = (BN * KCP + 63) / 64;    // direct-load instructions per K tile
  static constexpr int kVInst = (BN * VCP + 63) / 64;    // ... per V tile
  static constexpr int kKElems = kKInst * 64 * 8;
  static constexpr int kVElems = kVInst * 64 * 8;
  static constexpr int kStage = kKElems + kVElems;
  static constexpr int kKInstPerWave = (kKInst + kWaves - 1) / kWaves;
  static constexpr int kVInstPerWave = (kVInst + kWaves - 1) / kWaves;
  static constexpr int kEpiElems = kWaves * 32 * (D + 8);  // the epilogue's staged rows
  static constexpr int kLdsElems = 2 * kStage > kEpiElems ? 2 * kStage : kEpiElems;
  static_assert(D == 64 || D == 128 || D == 256, "the 16x16x32 kernel serves d = 64, 128 and 256");
  // Row strides of 8 (mod 16) dwords: for these read patterns (K: 16 rows x
  // 64 bytes per 16-byte read; V: 16 rows x 32 bytes per transpose read)
  // the counters show no bank conflicts in the tile loop, where a K stride
  // of 4 (mod 8) dwords cost about 4 conflict cycles per K read, and V
  // strides of 4 (mod 8) or 16 (mod 64) dwords 2 per transpose read.
  static_assert((KS / 2) % 16 == 8 && (VS / 2) % 16 == 8, "conflict-free row strides");
  static_assert((WIDE ? 1 : 2) * kLdsElems * 2 <= 160 * 1024, "workgroups per CU");
};

template <int D, bool BF16, bool CAUSAL, bool VARLEN = false, bool SPARSE = false, bool WIDE = false,
          bool WIN = false>
__global__ void __launch_bounds__((K16Cfg<D, WIDE>::kThreads), 2)
attn_fwd_k16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                    float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb, int total,
                    float c_log2, VarlenArgs va, BlockMaskArgs bm, int wl, int wr) {
  using C = K16Cfg<D, WIDE>;
  static_assert(!(SPARSE && VARLEN), "block sparsity is an instance of its own");
  static_assert(!WIDE || !SPARSE, "a mask block is one 128-row workgroup");
  static_assert(!WIN || (!SPARSE && !VARLEN && !WIDE), "the window is an instance of the batched layout");
  static_assert(kMaskBlock % C::BN == 0 && (!SPARSE || kMaskBlock == C::BM), "a mask block is whole tiles");
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NK4 = D / 32;   // 32-wide k-steps of S^T
  constexpr int NKB = BN / 16;  // 16-key blocks of S^T
  constexpr int NDB = D / 16;   // 16-dimension blocks of O^T
  constexpr int NKK = BN / 32;  // 32-key k-steps of the PV product

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;

  const WorkItem w = VARLEN ? map_workgroup_packed(blockIdx.x, nqb, Hq, va.pairs)
                           : map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;

  // First rows of this (b, head) in q/out and k/v, and of its lse row.
  int64_t q_row0 = (int64_t)w.b * Nq, k_row0 = (int64_t)w.b * Nk;
  int64_t lse_off = ((int64_t)w.b * Hq + w.hq) * Nq;
  if constexpr (VARLEN) {
    const int qs0 = min(max(va.cu_q[w.b], 0), va.total_q);
    const int ks0 = min(max(va.cu_k[w.b], 0), va.total_k);
    Nq = min(max(va.cu_q[w.b + 1], qs0), va.total_q) - qs0;
    Nk = min(max(va.cu_k[w.b + 1], ks0), va.total_k) - ks0;
    q_row0 = qs0;
    k_row0 = ks0;
    lse_off = (int64_t)w.hq * va.total_q + qs0;
    if (q0 >= Nq) return;  // the whole workgroup, before any barrier
  }
  const int diag = Nk - Nq;  // causal: key j visible to row i iff j <= i + diag

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const int64_t qh_off = q_row0 * q_rs + (int64_t)w.hq * D;
  const uint16_t* Kh = K + (k_row0 * Hkv + hkv) * D;
  const uint16_t* Vh = V + (k_row0 * Hkv + hkv) * D;

  // ---- Q^T fragments (B operand): block qb, k-step k4 holds dimensions
  // 32 k4 + 8 g .. + 7 of row qw0 + 16 qb + c; rows past Nq read as zero.
  u32x4_t qf[2][NK4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r0 = qw0 + 16 * qb;
    const rsrc_t qr = make_rsrc(Q + qh_off + (int64_t)r0 * q_rs, span_bytes(r0, 16, Nq, q_rs, D));
    const int voff = (int)(c * q_rs * 2) + 16 * g;
#pragma unroll
    for (int k4 = 0; k4 < NK4; ++k4) qf[qb][k4] = buf_load16(qr, voff + 64 * k4);
  }

  // ---- Key range of the workgroup and of this wave; tiles before nf are
  // visible to every row of the workgroup.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);
  // Sliding window (key j kept for row i iff i + diag - wl <= j <= i + diag
  // + wr; negative = unbounded): keys right of the last row's window are
  // never loaded, the walk starts at the tile of the first row's window
  // (jb), and a wave skips the tiles outside its own rows' windows.
  int jb = 0, w_begin = 0;
  if constexpr (WIN) {
    if (wr >= 0) {
      kv_end = min(kv_end, max(0, min(q0 + BM, Nq) + diag + wr));
      if (rows_end > qw0) w_end = min(w_end, max(0, rows_end + diag + wr));
    }
    if (wl >= 0) {
      jb = max(0, q0 + diag - wl) / BN;
      w_begin = qw0 + diag - wl;
    }
  }
  int nt = kv_end > jb * BN ? (kv_end - jb * BN + BN - 1) / BN : 0;
  int nf = Nk / BN;
  if (CAUSAL) nf = min(nf, max(0, (q0 + diag + 1) / BN));
  // With a window, tiles [t_lo, nf) (counted from jb) are the ones every row
  // of the workgroup sees whole; the ones before t_lo are cut by the
  // window's left edge.
  int t_lo = 0;
  if constexpr (WIN) {
    if (wr >= 0) nf = min(nf, max(0, (q0 + diag + wr + 1) / BN));
    if (wl >= 0) {
      const int q_last = min(q0 + BM, Nq) - 1;
      t_lo = max(0, (q_last + diag - wl + BN - 1) / BN - jb);
    }
    nf -= jb;
  }

  // ---- Block sparsity (attn_fwd_kernel's walk): the tiles of flagged key
  // blocks below kv_end, in key order; nt counts them and nf those every row
  // sees whole; unflagged tiles are never loaded.
  constexpr int TPB = kMaskBlock / BN;  // tiles per mask block
  int sp_chunk = 0, sp_blk = 0, sp_sub = TPB, sp_cur = 0, sp_nchunks = 0;
  uint64_t sp_bits = 0;
  const int nkb_eff = (kv_end + kMaskBlock - 1) / kMaskBlock;
  const int64_t sp_row = ((int64_t)w.b * bm.heads + (bm.heads == 1 ? 0 : w.hq)) * nqb + w.qblk;
  const rsrc_t sp_mr = make_rsrc(SPARSE ? bm.mask + sp_row * bm.nkb : nullptr, SPARSE ? nkb_eff : 0);
  if constexpr (SPARSE) {
    sp_nchunks = (nkb_eff + 63) / 64;
    const int full_blocks = nf / TPB, full_rem = nf % TPB;
    const int last = nkb_eff - 1;  // may hold fewer than TPB tiles
    const int last_tiles = (kv_end - kMaskBlock * last + BN - 1) / BN;
    int blocks = 0, nf_blocks = 0, sp_nf = 0;
    nt = 0;
    for (int ci = 0; ci < sp_nchunks; ++ci) {
      const uint64_t bits = flag_word(sp_mr, ci, 1, lane);
      if (ci == 0) sp_bits = bits;
      blocks += __builtin_popcountll(bits);
      const int below = full_blocks - 64 * ci;  // blocks of this chunk under full_blocks
      nf_blocks += __builtin_popcountll(below >= 64 ? bits : below <= 0 ? 0ull
                                        : bits & ((1ull << below) - 1));
      if (full_rem && below >= 0 && below < 64 && ((bits >> below) & 1)) sp_nf += full_rem;
      if (last / 64 == ci && ((bits >> (last % 64)) & 1)) nt -= TPB - last_tiles;
    }
    nt += TPB * blocks;
    nf = sp_nf + TPB * nf_blocks;
  }
  nf = min(max(nf, 0), nt);
  t_lo = min(t_lo, nf);
  // Start of the next visited tile (block sparsity only); called once per
  // tile, only while one is left, so a flagged block lies ahead.
  auto sparse_next = [&]() -> int {
    if (++sp_sub >= TPB) {
      while (sp_bits == 0 && sp_chunk + 1 < sp_nchunks) {
        ++sp_chunk;
        sp_bits = flag_word(sp_mr, sp_chunk, 1, lane);
      }
      sp_blk = 64 * sp_chunk + (sp_bits ? __builtin_ctzll(sp_bits) : 0);
      sp_bits &= sp_bits - 1;
      sp_sub = 0;
    }
    return sp_blk * kMaskBlock + sp_sub * BN;
  };

  // ---- Direct global->LDS tile loads: this wave issues the K (V) tile's
  // instructions j = wave, wave + kWaves, ...; lane -> 16-byte slot 64 j + lane ->
  // (row, chunk) of the padded layout.
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
  auto issue_tile = [&](int j0, uint16_t* stage) {
    const int bytes = span_bytes(j0, BN, Nk, kv_rs, D);
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, bytes);
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, bytes);
#pragma unroll
    for (int i = 0; i < C::kKInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      if (j < C::kKInst) buf_load_lds16(kr, stage + 512 * j, koff[i]);
    }
#pragma unroll
    for (int i = 0; i < C::kVInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      if (j < C::kVInst) buf_load_lds16(vr, stage + C::kKElems + 512 * j, voff[i]);
    }
  };

  // ---- Operand reads from LDS: K row 16 kb + c at column 32 k4 + 8 g; for
  // the transpose reads lane c of group g addresses V row 4 g + c / 4 (+ the
  // key step's base) at column 4 (c % 4) of the 16-column block, and receives
  // 4 consecutive keys at column c.
  const int k_rd = c * KS + 8 * g;
  const int v_rd = C::kKElems + (4 * g + (c >> 2)) * VS + 4 * (c & 3);

  // ---- Running state: two query rows per lane.
  f32x4_t oacc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x4_t{};
  float m[2] = {-INFINITY, -INFINITY};  // running max of s * c_log2 (log2 units)
  float lsum[2] = {0.f, 0.f};           // this lane's share of the running sums

  if constexpr (SPARSE) {
    if (nt > 0) sp_cur = sparse_next();
  }
  if (nt > 0) issue_tile(SPARSE ? sp_cur : jb * BN, smem);
  __builtin_amdgcn_s_waitcnt(0);  // Q fragments and tile 0 have landed
  __syncthreads();

  // S^T of the tile.  Per k-step the four K operands are read first and each
  // Q^T operand then feeds four consecutive MFMAs: the matrix cores' power,
  // and with it the clock this kernel runs at, depends on how many operands
  // change from one instruction to the next (measured: 4-5 % faster than
  // alternating the two query blocks, whose MFMAs share the K operand).
  auto compute_s = [&](const uint16_t* st, f32x4_t (&s)[2][NKB]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x4_t{};
#pragma unroll
    for (int k4 = 0; k4 < NK4; ++k4) {
      u32x4_t a[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) a[kb] = *reinterpret_cast<const u32x4_t*>(st + k_rd + kb * 16 * KS + 32 * k4);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = mfma_16x16x32<BF16>(a[kb], qf[qb][k4], s[qb][kb]);
    }
  };

  // Row maximum of block qb over the tile (in-lane, then across the four
  // lane groups); m is raised when it is exceeded by more than `threshold`,
  // and what was accumulated is rescaled.
  auto raise_max = [&](int qb, const f32x4_t (&s)[NKB], float threshold) {
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) tmax = max3(tmax, max3(s[kb][0], s[kb][1], s[kb][2]), s[kb][3]);
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

  // p = 2^(s*c - m) in place; returns this lane's sum of the unrounded p.
  auto exponentiate = [&](int qb, f32x4_t (&s)[NKB], auto m_finite) {
    const float mb = (decltype(m_finite)::value || m[qb] != -INFINITY) ? m[qb] : 0.f;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
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

  // Tile t (modes as in attn_fwd_kernel): kLean -- every key visible to
  // every row and m finite: exponentials against the current m, the maximum
  // path only when a partial row sum exceeds kSumLimit (S recomputed from the
  // K tile still in LDS); kFull -- every key visible, tile maximum first;
  // kMasked -- tile maximum first, masking where the tile crosses the causal
  // diagonal or the ragged end.
  constexpr int kLean = 0, kFull = 1, kMasked = 2;
  // The stage being filled and the one being read come in as
  // restrict-qualified parameters: the transpose reads of the current stage
  // then carry alias information that sets them apart from the next tile's
  // direct loads, so they need not wait for those loads (without it the
  // compiler waits for every outstanding direct-to-LDS load before the first
  // V^T read).  The wait at the end of the tile keeps the order.
  auto tile_body = [&](int t, auto mode, uint16_t* __restrict__ nxt, const uint16_t* __restrict__ st)
                       __attribute__((always_inline)) {
    constexpr int kMode = decltype(mode)::value;
    const int j0 = SPARSE ? sp_cur : (jb + t) * BN;
    if (t + 1 < nt) {
      int jn = j0 + BN;
      if constexpr (SPARSE) jn = sp_cur = sparse_next();
      issue_tile(jn, nxt);
    }

    // wave-uniform: skip tiles above this wave's diagonal (or outside its window)
    if (j0 < w_end && (!WIN || j0 + BN > w_begin)) {
      f32x4_t s[2][NKB];
      __builtin_amdgcn_s_setprio(1);
      compute_s(st, s);
      __builtin_amdgcn_s_setprio(0);
      bool need_mask = false;
      if constexpr (kMode == kLean) {
        float psum[2];
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          psum[qb] = exponentiate(qb, s[qb], std::true_type{});
          over = over || !(psum[qb] <= kSumLimit);
        }
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
          compute_s(st, s);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            raise_max(qb, s[qb], 0.0f);
            psum[qb] = exponentiate(qb, s[qb], std::true_type{});
          }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) lsum[qb] += psum[qb];
      } else {
        need_mask = kMode == kMasked && ((j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag));
        if constexpr (WIN) {
          if (wl >= 0 && j0 < qw0 + 31 + diag - wl) need_mask = true;
          if (wr >= 0 && j0 + BN - 1 > qw0 + diag + wr) need_mask = true;
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (need_mask) {
            const int my_q = qw0 + 16 * qb + c;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = j0 + 16 * kb + 4 * g + r;
                const int dist = my_q + diag - j;
                const bool vis = j < Nk && (!CAUSAL || dist >= 0) &&
                                 (!WIN || ((wl < 0 || dist <= wl) && (wr < 0 || -dist <= wr)));
                s[qb][kb][r] = vis ? s[qb][kb][r] : -INFINITY;
              }
            }
          }
          raise_max(qb, s[qb], kRescaleThreshold);
          lsum[qb] += exponentiate(qb, s[qb], std::false_type{});
        }
      }

      // O^T += V^T P^T; causal tiles that cross the diagonal feed P as
      // hi + lo halves (two MFMAs per step).
      auto pv_product = [&](auto with_lo) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          u32x4_t phi[2], plo[2];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            f32x8_t pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pv[e] = s[qb][2 * kk][e];
              pv[4 + e] = s[qb][2 * kk + 1][e];
            }
            phi[qb] = pack8<BF16>(pv);
            if constexpr (decltype(with_lo)::value) plo[qb] = pack8<BF16>(pv - unpack8<BF16>(phi[qb]));
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x2_t x0 = lds_read_tr4(st + v_rd + 32 * kk * VS + 16 * db);
            const u32x2_t x1 = lds_read_tr4(st + v_rd + (32 * kk + 16) * VS + 16 * db);
            const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              oacc[qb][db] = mfma_16x16x32<BF16>(a, phi[qb], oacc[qb][db]);
              if constexpr (decltype(with_lo)::value)
                oacc[qb][db] = mfma_16x16x32<BF16>(a, plo[qb], oacc[qb][db]);
            }
          }
        }
      };
      __builtin_amdgcn_s_setprio(1);
      // (with a block mask a row may keep only the keys of a ragged last
      // block, so its masked tiles take the lo half as well; a tile cut only
      // by the left edge of a window of at least 128 keys needs no lo half:
      // every row it holds sees at least that many keys)
      bool with_lo = (CAUSAL || SPARSE || WIN) && need_mask;
      if constexpr (WIN) {
        const bool right_edge = (CAUSAL && j0 + BN - 1 > qw0 + diag) ||
                                (wr >= 0 && j0 + BN - 1 > qw0 + diag + wr);
        if (wl >= 127 && !right_edge && j0 + BN <= Nk) with_lo = false;
      }
      if constexpr (D == 256) {
        // at d = 256 the lo half is a second sweep over the V^T blocks (read
        // again from LDS) after the hi one: a tile body with both halves
        // interleaved needs more registers than two workgroups per CU leave
        pv_product(std::false_type{});
        if (with_lo) {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            u32x4_t plo[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              f32x8_t pv;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                pv[e] = s[qb][2 * kk][e];
                pv[4 + e] = s[qb][2 * kk + 1][e];
              }
              plo[qb] = pack8<BF16>(pv - unpack8<BF16>(pack8<BF16>(pv)));
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const u32x2_t x0 = lds_read_tr4(st + v_rd + 32 * kk * VS + 16 * db);
              const u32x2_t x1 = lds_read_tr4(st + v_rd + (32 * kk + 16) * VS + 16 * db);
              const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) oacc[qb][db] = mfma_16x16x32<BF16>(a, plo[qb], oacc[qb][db]);
            }
          }
        }
      } else if (with_lo) {
        pv_product(std::true_type{});
      } else {
        pv_product(std::false_type{});
      }
      __builtin_amdgcn_s_setprio(0);
    }

    __builtin_amdgcn_s_waitcnt(0);  // tile t+1 has landed in LDS
    __syncthreads();
  };
  auto tile = [&](int t, auto mode) __attribute__((always_inline)) {
    tile_body(t, mode, smem + ((t + 1) & 1) * C::kStage, smem + (t & 1) * C::kStage);
  };
  using LeanMode = std::integral_constant<int, kLean>;
  using FullMode = std::integral_constant<int, kFull>;
  using MaskedMode = std::integral_constant<int, kMasked>;
  int t = 0;
  if constexpr (WIN) {
    for (; t < t_lo; ++t) tile(t, MaskedMode{});
  }
  if (t < nf) tile(t++, FullMode{});
  for (; t < nf; ++t) tile(t, LeanMode{});
  for (; t < nt; ++t) tile(t, MaskedMode{});

  // ---- Epilogue (every wave passed the last tile's barrier: no wave reads
  // the stages any more).  Rows are normalised, rounded and staged in this
  // wave's slice of LDS (row 16 qb + c, 4 dimensions per block and lane
  // group), then stored 16 contiguous bytes per lane.
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
  const rsrc_t orr = make_rsrc(O + qh_off + (int64_t)qw0 * q_rs, span_bytes(qw0, 32, Nq, q_rs, D));
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
