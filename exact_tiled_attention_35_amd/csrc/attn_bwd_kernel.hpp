// Exact attention backward for gfx950 (MI355X, CDNA4).
//
// Gradients of L = sum(dout * out) for out = softmax(Q K^T * scale) V, per
// (batch, query head), from the forward's out and logsumexp.  The pages state
// that the library computes gradients, that a deterministic backward pass
// exists (hysenlabs.com, "FlashAttention: exakte Attention-Kernel fuer CUDA
// und ROCm", section "Von 2.0 bis 2.7") and that its tests compare gradients
// with a reference (section "Tests, BSD-3-Clause und Zitierpraxis"); the
// formulas are the chain rule of the forward definition:
//
//   P = exp(S * scale - lse)            recomputed tile by tile, never stored
//   D_i = sum_c dO_ic O_ic              (= sum_j P_ij dP_ij)
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Two kernels, no atomics and no workspace, so results are bitwise
// reproducible run to run:
//  * attn_bwd_dq_kernel: one workgroup per 128 query rows of one (b, head),
//    4 waves x 32 rows, looping over key tiles.  Per tile and wave, on
//    v_mfma_f32_16x16x32 in 16 x 16 blocks (the layout of the forward's
//    attn_fwd_k16_kernel):
//        S^T  = K Q^T    (A = K rows from LDS, B = Q^T in VGPRs)
//        dP^T = V dO^T   (A = V rows from LDS, B = dO^T in VGPRs)
//        dQ^T += K^T dS^T (A = K^T by LDS transpose reads of the same K
//                          tile, B = dS^T packed from the accumulators)
//    Each lane holds two query rows (shared by its four lane groups), so
//    lse and D are two per-lane scalars.  The kernel first computes D for
//    its rows and stores it (the dK/dV kernel reads it).
//  * attn_bwd_dkdv_kernel: one workgroup per 128 keys of one (b, KV head),
//    4 waves x 32 keys (the plain d = 128 instance: 256 keys, 8 waves, one
//    workgroup per CU, so that each query tile is fetched from L2 once for
//    twice as many keys), looping over the query heads of the GQA group and
//    their query tiles of 32 rows.  The roles of queries and keys are
//    swapped relative to the dQ kernel; on v_mfma_f32_16x16x32:
//        S    = Q K^T    (A = Q rows from LDS, B = K^T in VGPRs)
//        dP   = dO V^T   (A = dO rows from LDS, B = V^T in VGPRs)
//        dV^T += dO^T P  (A = dO^T by LDS transpose reads of the same dO
//                         tile, B = P packed from the accumulators)
//        dK^T += Q^T dS  (A = Q^T likewise from the Q tile, B = dS packed)
//    Each lane owns two keys (shared by its four lane groups); lse and D of
//    the tile's query rows come from LDS.  The GQA group's sum happens in
//    registers.  At d = 128 the causal, score-variant and block-sparse
//    instances keep V^T (with ALiBi also the last K^T k-step) in LDS rather
//    than in registers.
// P is rounded to the element type for the dV product and dS for the dQ and
// dK products (fp32 accumulation throughout).
#pragma once

#include <type_traits>

#include "gfx950_ops.hpp"

namespace eta {

constexpr float kLog2e = 1.44269504088896340736f;

// Score-variant instances of the backward kernels (template argument MK):
// kModsOn marks one (the window is read at run time); kModsCap and
// kModsAlibi select the softcap and the ALiBi bias at compile time, so that
// each instance carries only the per-element work it needs.
constexpr int kModsOn = 1, kModsCap = 2, kModsAlibi = 4;

// Tiles read by the 16x16x32 products both as rows (16-byte reads, 16 rows
// x 64 bytes per read) and through transpose reads (16 rows x 32 bytes):
// rows padded to 8 (mod 16) dwords, free of bank conflicts for both (the
// forward's attn_fwd_k16_kernel measured it), so one copy of a tile serves
// both kinds of read.
template <int D>
struct Bwd16Layout {
  static constexpr int kChunks = D / 8;
  static constexpr int CP = kChunks + 2;   // 16-byte slots per row
  static constexpr int RS = 8 * CP;        // row stride, elements
  static_assert((RS / 2) % 16 == 8, "conflict-free row stride");
  template <int R>
  static constexpr int elems() { return ((R * CP + 63) / 64) * 512; }
};

template <int D>
struct DqCfg {
  static constexpr int kWaves = 4, kThreads = 256, BM = 128;
  // 32-key tiles keep the LDS of a workgroup under half of the CU's, so two
  // workgroups (two waves per SIMD) share a CU.
  static constexpr int BN = 32;  // keys per tile
  using L = Bwd16Layout<D>;
  static constexpr int kK = L::template elems<BN>();  // K: rows for S^T, transposed for dQ
  static constexpr int kV = kK;
  static constexpr int kStage = kK + kV;
  static constexpr int kLdsElems = 2 * kStage;
  static constexpr int kMinWavesPerEU = (D >= 256) ? 1 : 2;
};

template <int D, bool WIDE = false>
struct DkvCfg {
  // WIDE: 8 waves (256 keys) per workgroup, one workgroup per CU, so that
  // each query tile is fetched once for twice as many keys.
  static constexpr int kWaves = WIDE ? 8 : 4, kThreads = 64 * kWaves, BK = 32 * kWaves;
  static constexpr int BQ = 32;  // query rows per tile (two workgroups per CU at d <= 128)
  using L = Bwd16Layout<D>;
  static constexpr int kTile = L::template elems<BQ>();  // Q or dO: rows for S / dP, transposed for dK / dV
  static constexpr int kVec = 512;  // 1 KB: lse or D of the tile (64 lanes x 16 B)
  static constexpr int kStage = 2 * kTile + 2 * kVec;
  static constexpr int kLdsElems = 2 * kStage;
  static constexpr int kMinWavesPerEU = (D >= 256) ? 1 : 2;
  static_assert(BQ * 4 <= kVec * 2, "lse/D slots cover the tile");
};

// Direct-load slot offsets for an R-row tile with CP chunks per row and a
// global row stride of rs elements: of the W waves, this one issues
// instructions j = wave, wave + W, ...; lane -> slot 64 j + lane -> (row, chunk).
template <int R, int CP, int D, int NI, int W = 4>
__device__ __forceinline__ void tile_offsets(int wave, int lane, int64_t rs, int (&off)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int sl = 64 * (wave + W * i) + lane;
    const int row = min(sl / CP, R - 1), c = min(sl % CP, D / 8 - 1);
    off[i] = (int)(row * rs * 2) + 16 * c;
  }
}

template <int NINST, int NI, int W = 4>
__device__ __forceinline__ void tile_issue(rsrc_t r, uint16_t* dst, int wave, const int (&off)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = wave + W * i;
    if (j < NINST) buf_load_lds16(r, dst + 512 * j, off[i]);
  }
}

// ---------------------------------------------------------------------------
// dQ (and D).
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL, bool SPARSE = false, bool VARLEN = false, int MK = 0>
__global__ void __launch_bounds__(DqCfg<D>::kThreads, DqCfg<D>::kMinWavesPerEU)
attn_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
                   const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
                   uint16_t* __restrict__ dQ, float* __restrict__ Dlt, int Hq, int Hkv, int Nq,
                   int Nk, int nqb, int total, float scale, float c_log2, BlockMaskArgs bm,
                   VarlenArgs va, ScoreMods mods) {
  constexpr bool MODS = MK != 0;
  constexpr bool kCap = (MK & kModsCap) != 0, kAlibi = (MK & kModsAlibi) != 0;
  static_assert((int)SPARSE + (int)VARLEN + (int)MODS <= 1, "one instance per extension");
  using C = DqCfg<D>;
  static_assert(kMaskBlock == C::BM && kMaskBlock % C::BN == 0, "a mask block is whole tiles");
  using L = typename C::L;
  constexpr int BN = C::BN, BM = C::BM, RS = L::RS;
  constexpr int NK4 = D / 32;  // 32-wide k-steps of S^T and dP^T
  constexpr int NDB = D / 16;  // 16-dimension blocks of dQ^T
  static_assert(BN == 32, "one 32-key step of the dQ product per tile");
  constexpr int kInst = C::kK / 512, kPW = (kInst + 3) / 4;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  // Lane l: group g = l / 16, c = l % 16.  S^T, dP^T and dQ^T are held in
  // 16 x 16 blocks (v_mfma_f32_16x16x32): block (qb, kb) register r of S^T
  // is key 16 kb + 4 g + r against query qw0 + 16 qb + c, so each lane owns
  // the two query rows qw0 + c and qw0 + 16 + c (shared by the four lane
  // groups); dQ^T block (qb, db) register r is dimension 16 db + 4 g + r.
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const WorkItem w = VARLEN ? map_workgroup_packed(blockIdx.x, nqb, Hq, va.pairs)
                           : map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM, qw0 = q0 + wave * 32;
  // First rows of this (b, head) in q-shaped and k-shaped tensors, and of
  // its lse / delta row; packed sequences take theirs from the prefix sums.
  int64_t q_row0 = (int64_t)w.b * Nq, k_row0 = (int64_t)w.b * Nk;
  int64_t vec_row0 = ((int64_t)w.b * Hq + w.hq) * Nq;
  if constexpr (VARLEN) {
    const int qs0 = min(max(va.cu_q[w.b], 0), va.total_q);
    const int ks0 = min(max(va.cu_k[w.b], 0), va.total_k);
    Nq = min(max(va.cu_q[w.b + 1], qs0), va.total_q) - qs0;
    Nk = min(max(va.cu_k[w.b + 1], ks0), va.total_k) - ks0;
    q_row0 = qs0;
    k_row0 = ks0;
    vec_row0 = (int64_t)w.hq * va.total_q + qs0;
    if (q0 >= Nq) return;  // the whole workgroup, before any barrier
  }
  const int diag = Nk - Nq;

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const int64_t qo_off = (q_row0 + qw0) * q_rs + (int64_t)w.hq * D;
  const uint16_t* Kh = K + (k_row0 * Hkv + hkv) * D;
  const uint16_t* Vh = V + (k_row0 * Hkv + hkv) * D;

  // Q^T and dO^T fragments (B operands) of the two row blocks, O for D.
  // Rows >= Nq read as 0.
  const int rspan = span_bytes(qw0, 32, Nq, q_rs, D);
  const rsrc_t qr = make_rsrc(Q + qo_off, rspan);
  const rsrc_t dor = make_rsrc(dO + qo_off, rspan);
  const rsrc_t orr = make_rsrc(O + qo_off, rspan);
  u32x4_t qf[2][NK4], df[2][NK4];
  float Di[2], lse2[2];
  const int nrows = max(0, min(32, Nq - qw0));
  const int64_t vec_off = vec_row0 + qw0;
  const rsrc_t lr = make_rsrc(LSE + vec_off, nrows * 4);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int fvoff = (int)((16 * qb + c) * q_rs * 2) + 16 * g;
    float dsum = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < NK4; ++k4) {
      qf[qb][k4] = buf_load16(qr, fvoff + 64 * k4);
      df[qb][k4] = buf_load16(dor, fvoff + 64 * k4);
      const u32x4_t o = buf_load16(orr, fvoff + 64 * k4);
      const f32x8_t a = unpack8<BF16>(df[qb][k4]), b = unpack8<BF16>(o);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf(a[e], b[e], dsum);
    }
    dsum += __shfl_xor(dsum, 16);
    Di[qb] = dsum + __shfl_xor(dsum, 32);
    // lse in log2 units; an empty row (lse = -inf) has every key masked.
    lse2[qb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, 4 * (16 * qb + c), 0, 0)) * kLog2e;
  }
  if (g == 0) {
    const rsrc_t dr = make_rsrc(Dlt + vec_off, nrows * 4);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) buf_store4(Di[qb], dr, 4 * (16 * qb + c));
  }

  // Key range of the workgroup and of this wave.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);
  // Window: keys right of the last row's window are never loaded, tiles left
  // of the first row's window are skipped (jb = first tile), and a wave
  // skips tiles outside its own rows' windows.
  int jb = 0, w_begin = 0;
  float slope = 0.f;
  if constexpr (MODS) {
    if (mods.right >= 0) {
      kv_end = min(kv_end, max(0, min(q0 + BM, Nq) + diag + mods.right));
      if (rows_end > qw0) w_end = min(w_end, max(0, rows_end + diag + mods.right));
    }
    if (mods.left >= 0) {
      jb = max(0, q0 + diag - mods.left) / BN;
      w_begin = qw0 + diag - mods.left;
    }
    nt = kv_end > jb * BN ? (kv_end - jb * BN + BN - 1) / BN : 0;
    if constexpr (kAlibi) slope = mods.slopes[w.hq];
  }
  // Score variants in log2 units (softcap: exp2 argument 2 x log2e with
  // x = sigma s / cap, output scale cap log2e), and the distances
  // dist = row + diag - j each row sees as one interval [vis_lo, vis_hi]
  // (keys past the end, causal, window).
  const float sigma_l2 = mods.sigma * kLog2e, slope_l2 = slope * kLog2e, cap_l2 = mods.cap * kLog2e;
  const float cap_in = kCap ? mods.sigma * __builtin_amdgcn_rcpf(mods.cap) * (2.0f * kLog2e) : 0.f;
  int lo_i[2], hi_i = 1 << 30;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    lo_i[qb] = qw0 + 16 * qb + c - Nq + 1;
    if (CAUSAL) lo_i[qb] = max(lo_i[qb], 0);
    if (MODS && mods.right >= 0) lo_i[qb] = max(lo_i[qb], -mods.right);
  }
  if (MODS && mods.left >= 0) hi_i = mods.left;

  // Block sparsity: the tiles of the flagged key blocks below kv_end, in key
  // order, as in the forward (flags read 64 blocks per ballot; tiles of
  // dropped blocks are never loaded).
  constexpr int TPB = kMaskBlock / BN;
  int sp_chunk = 0, sp_blk = 0, sp_sub = TPB, sp_nchunks = 0, sp_cur = 0;
  uint64_t sp_bits = 0;
  const int nkb_eff = kv_end > 0 ? (kv_end + kMaskBlock - 1) / kMaskBlock : 0;
  const int64_t sp_row = ((int64_t)w.b * bm.heads + (bm.heads == 1 ? 0 : w.hq)) * nqb + w.qblk;
  const rsrc_t sp_mr = make_rsrc(SPARSE ? bm.mask + sp_row * bm.nkb : nullptr, SPARSE ? nkb_eff : 0);
  if constexpr (SPARSE) {
    sp_nchunks = (nkb_eff + 63) / 64;
    const int last = nkb_eff - 1;  // may hold fewer than TPB tiles
    const int last_tiles = (kv_end - kMaskBlock * last + BN - 1) / BN;
    int blocks = 0;
    nt = 0;
    for (int ci = 0; ci < sp_nchunks; ++ci) {
      const uint64_t bits = flag_word(sp_mr, ci, 1, lane);
      if (ci == 0) sp_bits = bits;
      blocks += __builtin_popcountll(bits);
      if (last / 64 == ci && ((bits >> (last % 64)) & 1)) nt -= TPB - last_tiles;
    }
    nt += TPB * blocks;
  }
  // Start of the next visited tile; called only while one is left.
  auto sparse_next = [&]() -> int {
    if (++sp_sub >= TPB) {
      while (sp_bits == 0 && sp_chunk + 1 < sp_nchunks) sp_bits = flag_word(sp_mr, ++sp_chunk, 1, lane);
      sp_blk = 64 * sp_chunk + (sp_bits ? __builtin_ctzll(sp_bits) : 0);
      sp_bits &= sp_bits - 1;
      sp_sub = 0;
    }
    return sp_blk * kMaskBlock + sp_sub * BN;
  };

  // K and V tiles, one padded row-major copy each.
  int toff[kPW];
  tile_offsets<BN, L::CP, D>(wave, lane, kv_rs, toff);
  auto issue_tile = [&](int j0, uint16_t* st) {
    const int bytes = span_bytes(j0, BN, Nk, kv_rs, D);
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, bytes);
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, bytes);
    tile_issue<kInst>(kr, st, wave, toff);
    tile_issue<kInst>(vr, st + C::kK, wave, toff);
  };

  // A operands: K / V row 16 kb + c at column 32 k4 + 8 g (16-byte reads);
  // K^T for the dQ product by transpose reads: lane c of group g addresses
  // K row 4 g + c / 4 (+ 16) at column 4 (c % 4) of a 16-column block and
  // receives 4 consecutive keys at column c.
  const int r_rd = c * RS + 8 * g;
  const int t_rd = (4 * g + (c >> 2)) * RS + 4 * (c & 3);

  f32x4_t acc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4_t{};

  if constexpr (SPARSE) {
    if (nt > 0) sp_cur = sparse_next();
  }
  if (nt > 0) issue_tile(SPARSE ? sp_cur : jb * BN, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int j0 = SPARSE ? sp_cur : (jb + t) * BN;
    if (t + 1 < nt) {
      int jn = j0 + BN;
      if constexpr (SPARSE) jn = sp_cur = sparse_next();
      issue_tile(jn, smem + ((t + 1) & 1) * C::kStage);
    }
    const uint16_t* kt = smem + (t & 1) * C::kStage;
    const uint16_t* vt = kt + C::kK;

    if (j0 < w_end && (!MODS || j0 + BN > w_begin)) {
      f32x4_t s[2][2], dp[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[qb][kb] = dp[qb][kb] = f32x4_t{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k4 = 0; k4 < NK4; ++k4) {
        u32x4_t ak[2], av[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ak[kb] = *reinterpret_cast<const u32x4_t*>(kt + r_rd + kb * 16 * RS + 32 * k4);
          av[kb] = *reinterpret_cast<const u32x4_t*>(vt + r_rd + kb * 16 * RS + 32 * k4);
        }
        // each Q^T (dO^T) operand feeds two consecutive MFMAs
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) s[qb][kb] = mfma_16x16x32<BF16>(ak[kb], qf[qb][k4], s[qb][kb]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) dp[qb][kb] = mfma_16x16x32<BF16>(av[kb], df[qb][k4], dp[qb][kb]);
      }
      __builtin_amdgcn_s_setprio(0);
      // dS^T = P^T (dP^T - D), P^T = 2^(s c - lse2); keys past the end and
      // (causal) above the diagonal get P = 0.
      const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag);
      if constexpr (MODS) {
        // Score variants on every element: t = sigma s, softcapped, minus the
        // ALiBi bias (log2 units); dS carries the softcap's derivative
        // 1 - tanh^2.  Only tiles cut by the end, the diagonal or the window
        // test distances.
        const bool mmask = need_mask || (mods.left >= 0 && qw0 + 31 + diag - j0 > mods.left) ||
                           (mods.right >= 0 && j0 + BN - 1 - qw0 - diag > mods.right);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int fd = qw0 + 16 * qb + c + diag - j0 - 4 * g;  // distance at kb = r = 0
          const float fdf = (float)fd;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // distance as fp32 (exact: far below 2^24)
              const float d = fdf - (float)(16 * kb + r);
              const float base = kAlibi ? __builtin_fmaf(-slope_l2, __builtin_fabsf(d), -lse2[qb]) : -lse2[qb];
              float p, gd = 1.f;
              if constexpr (kCap) {
                const float th = __builtin_fmaf(
                    -2.f, __builtin_amdgcn_rcpf(exp2_fast(s[qb][kb][r] * cap_in) + 1.f), 1.f);
                gd = __builtin_fmaf(-th, th, 1.f);
                p = exp2_fast(__builtin_fmaf(th, cap_l2, base));
              } else {
                p = exp2_fast(__builtin_fmaf(s[qb][kb][r], sigma_l2, base));
              }
              const float tv = p * (dp[qb][kb][r] - Di[qb]);
              s[qb][kb][r] = kCap ? tv * gd : tv;
            }
          }
          if (mmask) {
            // Element offset o = 16 kb + r is visible iff fd - o lies in
            // [lo_i, hi_i]; a select, so that an infinite or NaN value of a
            // hidden element goes away.
            const int o_lo = fd - hi_i, o_hi = fd - lo_i[qb];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int o = 16 * kb + r;
                s[qb][kb][r] = (o >= o_lo && o <= o_hi) ? s[qb][kb][r] : 0.f;
              }
            }
          }
        }
      } else {
        // Tiles cut by the end or the diagonal test every element; the
        // others take a body without the test (as one body, the compiler
        // turns the test into selects that every tile pays for).
        auto p_ds = [&](auto masked) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                float p = exp2_fast(__builtin_fmaf(s[qb][kb][r], c_log2, -lse2[qb]));
                if constexpr (decltype(masked)::value) {
                  const int j = j0 + 16 * kb + 4 * g + r;
                  const bool vis = j < Nk && (!CAUSAL || j <= qw0 + 16 * qb + c + diag);
                  p = vis ? p : 0.f;
                }
                s[qb][kb][r] = p * (dp[qb][kb][r] - Di[qb]);
              }
            }
          }
        };
        if (need_mask)
          p_ds(std::true_type{});
        else
          p_ds(std::false_type{});
      }
      // dQ^T += K^T dS^T: lane group g feeds the keys {4 g .. 4 g + 3,
      // 16 + 4 g .. 16 + 4 g + 3}, the registers of dS^T blocks kb = 0, 1;
      // each K^T operand feeds two consecutive MFMAs (the two row blocks).
      u32x4_t b[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x8_t pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = s[qb][0][e];
          pv[4 + e] = s[qb][1][e];
        }
        b[qb] = pack8<BF16>(pv);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x2_t x0 = lds_read_tr4(kt + t_rd + 16 * db);
        const u32x2_t x1 = lds_read_tr4(kt + t_rd + 16 * RS + 16 * db);
        const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[qb][db] = mfma_16x16x32<BF16>(a, b[qb], acc[qb][db]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // dQ = scale * acc, rounded; rows >= Nq fall outside the store range.
  const rsrc_t dqr = make_rsrc(dQ + qo_off, rspan);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int ovoff = (int)((16 * qb + c) * q_rs * 2) + 8 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db) buf_store8(pack4<BF16>(acc[qb][db] * scale), dqr, ovoff + 32 * db);
  }
}

// ---------------------------------------------------------------------------
// dK and dV.
// ---------------------------------------------------------------------------
// blockIdx -> (b, KV head, key block); causal launches run the first key
// blocks (which see the most query rows) first, as the grid is dispatched in
// order.
__device__ __forceinline__ WorkItem map_key_block(int wg, int total, int nkb, int Hkv) {
  int lid = wg;
  if ((total & 7) == 0) lid = (wg & 7) * (total >> 3) + (wg >> 3);
  WorkItem w;
  w.qblk = lid % nkb;
  const int bh = lid / nkb;
  w.hq = bh % Hkv;
  w.b = bh / Hkv;
  return w;
}

template <int D, bool BF16, bool CAUSAL, bool SPARSE = false, bool VARLEN = false, int MK = 0, bool WIDE = false>
__global__ void __launch_bounds__((DkvCfg<D, WIDE>::kThreads), (DkvCfg<D, WIDE>::kMinWavesPerEU))
attn_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ Dlt,
                     uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv,
                     int Nq, int Nk, int nkb, int total, float scale, float c_log2,
                     BlockMaskArgs bm, VarlenArgs va, ScoreMods mods) {
  constexpr bool MODS = MK != 0;
  constexpr bool kCap = (MK & kModsCap) != 0, kAlibi = (MK & kModsAlibi) != 0;
  static_assert((int)SPARSE + (int)VARLEN + (int)MODS <= 1, "one instance per extension");
  using C = DkvCfg<D, WIDE>;
  static_assert(!WIDE || (!SPARSE && !VARLEN && !MODS && !CAUSAL), "the wide workgroup serves the plain instance");
  static_assert((!SPARSE || kMaskBlock == C::BK) && kMaskBlock % C::BQ == 0, "a mask block is whole tiles");
  using L = typename C::L;
  constexpr int BQ = C::BQ, BK = C::BK, RS = L::RS;
  constexpr int NK4 = D / 32;  // 32-wide k-steps of S and dP
  constexpr int NDB = D / 16;  // 16-dimension blocks of dK^T and dV^T
  static_assert(BQ == 32, "one 32-row step of the dK / dV products per tile");
  constexpr int W = C::kWaves;
  constexpr int kInst = C::kTile / 512, kPW = (kInst + W - 1) / W;
  // The causal, score-variant and block-sparse instances at d = 128 carry
  // more per-lane state than the 256 registers of two waves per SIMD leave
  // room for; there the V^T fragments sit in LDS (one 16-byte slot per lane
  // and fragment, conflict-free reads) instead of being spilled to scratch,
  // whose reloads would wait for the next tile's loads.  With the ALiBi bias
  // the last 32 dimensions of K^T go there too.
  constexpr bool kStashV = (MODS || SPARSE || CAUSAL) && D == 128;
  constexpr int kStashK = (kAlibi && D == 128) ? 1 : 0;  // K^T k-steps, from the last
  constexpr int kStashWave = 2 * (NK4 + kStashK) * 64 * 8;  // elements per wave
  constexpr int kStashElems = kStashV ? W * kStashWave : 0;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems + kStashElems];

  // Lane l: group g = l / 16, c = l % 16.  S, dP and dK^T, dV^T are held in
  // 16 x 16 blocks (v_mfma_f32_16x16x32): block (qb, kb) register r of S is
  // query row i0 + 16 qb + 4 g + r against key kw0 + 16 kb + c, so each lane
  // owns the two keys kw0 + c and kw0 + 16 + c (shared by the four lane
  // groups); dK^T / dV^T block (db, kb) register r is dimension
  // 16 db + 4 g + r of key kw0 + 16 kb + c.
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  // (w.hq is the KV head here, w.qblk the key block.)
  const WorkItem w = VARLEN ? map_workgroup_packed(blockIdx.x, nkb, Hkv, va.pairs)
                           : map_key_block(blockIdx.x, total, nkb, Hkv);
  const int G = Hq / Hkv;
  const int k0 = w.qblk * BK, kw0 = k0 + wave * 32;
  // First rows of this batch entry (or packed sequence) in q-shaped and
  // k-shaped tensors; lse / delta of query head h start at vec_row0(h).
  int64_t q_row0 = (int64_t)w.b * Nq, k_row0 = (int64_t)w.b * Nk;
  int64_t vec_stride = Nq, vec_first = (int64_t)w.b * Hq * Nq;
  if constexpr (VARLEN) {
    const int qs0 = min(max(va.cu_q[w.b], 0), va.total_q);
    const int ks0 = min(max(va.cu_k[w.b], 0), va.total_k);
    Nq = min(max(va.cu_q[w.b + 1], qs0), va.total_q) - qs0;
    Nk = min(max(va.cu_k[w.b + 1], ks0), va.total_k) - ks0;
    q_row0 = qs0;
    k_row0 = ks0;
    vec_stride = va.total_q;
    vec_first = qs0;
    if (k0 >= Nk) return;  // the whole workgroup, before any barrier
  }
  auto vec_row0 = [&](int h) { return vec_first + (int64_t)h * vec_stride; };
  const int diag = Nk - Nq;  // key j visible to query i iff j <= i + diag

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const int64_t kv_off = (k_row0 + kw0) * kv_rs + (int64_t)w.hq * D;

  // K^T and V^T fragments of this wave's two key blocks (B operands): key
  // kw0 + 16 kb + c, dimensions 32 k4 + 8 g .. + 7.
  const int kspan = span_bytes(kw0, 32, Nk, kv_rs, D);
  const rsrc_t kr = make_rsrc(K + kv_off, kspan);
  const rsrc_t vr = make_rsrc(V + kv_off, kspan);
  u32x4_t kf[2][NK4], vf[2][NK4];
  uint16_t* const vstash = smem + C::kLdsElems + wave * kStashWave + 8 * lane;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int fvoff = (int)((16 * kb + c) * kv_rs * 2) + 16 * g;
#pragma unroll
    for (int k4 = 0; k4 < NK4; ++k4) {
      kf[kb][k4] = buf_load16(kr, fvoff + 64 * k4);
      vf[kb][k4] = buf_load16(vr, fvoff + 64 * k4);
      if constexpr (kStashV) *reinterpret_cast<u32x4_t*>(vstash + 512 * (kb * NK4 + k4)) = vf[kb][k4];
      if constexpr (kStashK > 0)
        if (k4 >= NK4 - kStashK)
          *reinterpret_cast<u32x4_t*>(vstash + 512 * (2 * NK4 + kb * kStashK + k4 - (NK4 - kStashK))) = kf[kb][k4];
    }
  }

  // Query tiles: every query head of the group, query rows from the first
  // tile any key of the workgroup sees (causal) to the end.
  const int nqt_all = (Nq + BQ - 1) / BQ;
  int qt_begin = 0;
  if (CAUSAL) qt_begin = min(nqt_all, max(0, k0 - diag) / BQ);
  int nqt = nqt_all - qt_begin;
  if constexpr (MODS) {
    // Window: query rows whose window holds a key of this block.
    if (mods.right >= 0) qt_begin = max(qt_begin, min(nqt_all, max(0, k0 - diag - mods.right) / BQ));
    int qt_end = nqt_all;
    if (mods.left >= 0) {
      const int i_max = k0 + BK - 1 - diag + mods.left;
      qt_end = i_max < 0 ? 0 : min(nqt_all, i_max / BQ + 1);
    }
    nqt = max(0, qt_end - qt_begin);
  }
  int nsteps = (k0 < Nk) ? G * nqt : 0;

  // Block sparsity: for each query head of the group, the query tiles of the
  // query blocks whose flag with this key block is set (a column of the
  // mask: stride nkb bytes), within [qt_begin, nqt_all), head by head in
  // block order -- the plain kernel's step order with dropped steps left out.
  constexpr int TPQ = kMaskBlock / BQ;  // query tiles per mask block
  const int nqbm = (Nq + kMaskBlock - 1) / kMaskBlock;
  const int qb_lo = qt_begin / TPQ, qb_hi = (nqt_all - 1) / TPQ;
  const int c_lo = qb_lo / 64, c_hi = max(qb_hi, 0) / 64;
  auto column = [&](int gi) {
    const int hm = bm.heads == 1 ? 0 : w.hq * G + gi;
    const int64_t base = ((int64_t)w.b * bm.heads + hm) * nqbm * bm.nkb + w.qblk;
    return make_rsrc(SPARSE ? bm.mask + base : nullptr, SPARSE && nqbm > 0 ? (nqbm - 1) * bm.nkb + 1 : 0);
  };
  // flags of query blocks [64 ch, 64 ch + 64) of head gi, limited to [qb_lo, qb_hi]
  auto range_word = [&](int gi, int ch) -> uint64_t {
    uint64_t bits = flag_word(column(gi), ch, bm.nkb, lane);
    if (ch == c_lo) bits &= ~0ull << (qb_lo % 64);
    if (ch == c_hi && qb_hi % 64 != 63) bits &= (1ull << (qb_hi % 64 + 1)) - 1;
    return bits;
  };
  int sp_gi = 0, sp_chunk = c_lo, sp_qt = 0, sp_qt_end = 0, sp_h = 0, sp_i0 = 0;
  uint64_t sp_bits = 0;
  if constexpr (SPARSE) {
    nsteps = 0;
    if (k0 < Nk && nqt > 0) {
      for (int gi = 0; gi < G; ++gi) {
        for (int ch = c_lo; ch <= c_hi; ++ch) {
          const uint64_t bits = range_word(gi, ch);
          if (gi == 0 && ch == c_lo) sp_bits = bits;
          nsteps += TPQ * __builtin_popcountll(bits);
          if (qb_lo / 64 == ch && ((bits >> (qb_lo % 64)) & 1)) nsteps -= qt_begin - TPQ * qb_lo;
          if (qb_hi / 64 == ch && ((bits >> (qb_hi % 64)) & 1)) nsteps -= TPQ * qb_hi + TPQ - nqt_all;
        }
      }
    }
  }
  // The next visited step (head and query tile); called only while one is left.
  auto sparse_next = [&]() {
    if (++sp_qt >= sp_qt_end) {
      for (int guard = 0; sp_bits == 0 && guard < G * (c_hi - c_lo + 1); ++guard) {
        if (++sp_chunk > c_hi) {
          sp_chunk = c_lo;
          if (++sp_gi >= G) sp_gi = G - 1;
        }
        sp_bits = range_word(sp_gi, sp_chunk);
      }
      const int qbm = 64 * sp_chunk + (sp_bits ? __builtin_ctzll(sp_bits) : qb_lo % 64);
      sp_bits &= sp_bits - 1;
      sp_qt = max(TPQ * qbm, qt_begin);
      sp_qt_end = min(TPQ * qbm + TPQ, nqt_all);
    }
    sp_h = w.hq * G + sp_gi;
    sp_i0 = sp_qt * BQ;
  };
  // First query row this wave's keys see (causal), for skipping whole tiles.
  const int w_first = CAUSAL ? kw0 - diag : -(1 << 30);
  // Score variants in log2 units (as in the dQ kernel), and the distances
  // dist = i + diag - j each of this lane's keys sees as one interval
  // [lo_i, hi_i[kb]] (rows past the end, causal, window; none for keys past
  // the end).
  const float sigma_l2 = mods.sigma * kLog2e, cap_l2 = mods.cap * kLog2e;
  const float cap_in = kCap ? mods.sigma * __builtin_amdgcn_rcpf(mods.cap) * (2.0f * kLog2e) : 0.f;
  int lo_i = CAUSAL ? 0 : -(1 << 29), hi_i[2];
  if (MODS && mods.right >= 0) lo_i = max(lo_i, -mods.right);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = kw0 + 16 * kb + c;
    hi_i[kb] = Nk - j - 1;
    if (MODS && mods.left >= 0) hi_i[kb] = min(hi_i[kb], mods.left);
    if (j >= Nk) hi_i[kb] = -(1 << 30);
  }
  const bool w_live = kw0 < Nk;

  // Q and dO tiles, one padded row-major copy each, then lse and D.
  int toff[kPW];
  tile_offsets<BQ, L::CP, D, kPW, W>(wave, lane, q_rs, toff);
  // Step s: query head hq = hkv*G + s / nqt, query tile qt_begin + s % nqt.
  auto step_rows = [&](int s) { return (qt_begin + s % nqt) * BQ; };
  auto issue_step = [&](int s, uint16_t* st) {
    const int h = SPARSE ? sp_h : w.hq * G + s / nqt;
    const int i0 = SPARSE ? sp_i0 : step_rows(s);
    const int64_t off = (q_row0 + i0) * q_rs + (int64_t)h * D;
    const int bytes = span_bytes(i0, BQ, Nq, q_rs, D);
    tile_issue<kInst, kPW, W>(make_rsrc(Q + off, bytes), st, wave, toff);
    tile_issue<kInst, kPW, W>(make_rsrc(dO + off, bytes), st + C::kTile, wave, toff);
    if (wave == 0) {
      const int64_t voff = vec_row0(h) + i0;
      const int vb = max(0, min(BQ, Nq - i0)) * 4;
      buf_load_lds16(make_rsrc(LSE + voff, vb), st + 2 * C::kTile, 16 * lane);
      buf_load_lds16(make_rsrc(Dlt + voff, vb), st + 2 * C::kTile + C::kVec, 16 * lane);
    }
  };

  // A operands: Q / dO row 16 qb + c at column 32 k4 + 8 g (16-byte reads);
  // Q^T and dO^T for the dK / dV products by transpose reads: lane c of
  // group g addresses row 4 g + c / 4 (+ 16) at column 4 (c % 4) of a
  // 16-column block and receives 4 consecutive rows at column c.
  const int r_rd = c * RS + 8 * g;
  const int t_rd = (4 * g + (c >> 2)) * RS + 4 * (c & 3);

  f32x4_t dk[NDB][2], dv[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dk[db][kb] = dv[db][kb] = f32x4_t{};

  if constexpr (SPARSE) {
    if (nsteps > 0) sparse_next();
  }
  if (nsteps > 0) issue_step(0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int cur_i0 = SPARSE ? sp_i0 : step_rows(s);
    float slope = 0.f;
    if constexpr (kAlibi) slope = mods.slopes[w.hq * G + s / nqt];
    if (s + 1 < nsteps) {
      if constexpr (SPARSE) sparse_next();
      issue_step(s + 1, smem + ((s + 1) & 1) * C::kStage);
    }
    const uint16_t* st = smem + (s & 1) * C::kStage;
    const uint16_t* qt = st;
    const uint16_t* dt = st + C::kTile;
    const float* lse_t = reinterpret_cast<const float*>(st + 2 * C::kTile);
    const float* dlt_t = lse_t + C::kVec / 2;
    const int i0 = cur_i0;

    bool in_window = true;
    if constexpr (MODS) {
      if (mods.right >= 0 && kw0 > i0 + BQ - 1 + diag + mods.right) in_window = false;
      if (mods.left >= 0 && kw0 + 31 < i0 + diag - mods.left) in_window = false;
    }
    if (w_live && i0 + BQ - 1 >= w_first && in_window) {  // wave-uniform: some pair visible
      f32x4_t sc[2][2], dp[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[qb][kb] = dp[qb][kb] = f32x4_t{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k4 = 0; k4 < NK4; ++k4) {
        u32x4_t aq[2], ad[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          aq[qb] = *reinterpret_cast<const u32x4_t*>(qt + r_rd + qb * 16 * RS + 32 * k4);
          ad[qb] = *reinterpret_cast<const u32x4_t*>(dt + r_rd + qb * 16 * RS + 32 * k4);
        }
        // each K^T (V^T) operand feeds two consecutive MFMAs
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4_t bk =
              k4 >= NK4 - kStashK
                  ? *reinterpret_cast<const u32x4_t*>(vstash + 512 * (2 * NK4 + kb * kStashK + k4 - (NK4 - kStashK)))
                  : kf[kb][k4];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) sc[qb][kb] = mfma_16x16x32<BF16>(aq[qb], bk, sc[qb][kb]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4_t bv = kStashV ? *reinterpret_cast<const u32x4_t*>(vstash + 512 * (kb * NK4 + k4)) : vf[kb][k4];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) dp[qb][kb] = mfma_16x16x32<BF16>(ad[qb], bv, dp[qb][kb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // P = 2^(s c - lse2) and dS = P (dP - D) for the rows this lane's
      // registers hold: row i0 + 16 qb + 4 g + r.  Rows past Nq read zero Q
      // and dO rows and lse = D = 0: their P is 1 and their dS 0, and they
      // add nothing to dV^T (dO rows zero) or dK^T (Q rows zero); keys past
      // Nk are never stored.  So only causal tiles that cross the diagonal
      // need masking (the score variants test their window and ragged ends
      // below).
      const bool need_mask = MODS ? (i0 + BQ > Nq) || (CAUSAL && i0 + diag < kw0 + 31)
                                  : (CAUSAL && i0 + diag < kw0 + 31);
      // dV^T += dO^T P and dK^T += Q^T dS take P and dS of key block kb as
      // one packed operand each: query rows {4 g .. 4 g + 3} (block qb = 0)
      // then {16 + 4 g .. 16 + 4 g + 3} (qb = 1).
      u32x4_t pb[2], sb[2];
      auto pack_kb = [&](int kb) {
        f32x8_t pv, sv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = sc[0][kb][e];
          pv[4 + e] = sc[1][kb][e];
          sv[e] = dp[0][kb][e];
          sv[4 + e] = dp[1][kb][e];
        }
        pb[kb] = pack8<BF16>(pv);
        sb[kb] = pack8<BF16>(sv);
      };
      if constexpr (MODS) {
        // The score variants, as in the dQ kernel; distance
        // d = i + diag - j = fd[kb] + 16 qb + r.  One key block at a time,
        // packed before the next starts, so that the softcap's temporaries
        // of both blocks are never live together.
        const bool mmask = need_mask || (mods.left >= 0 && i0 + BQ - 1 + diag - kw0 > mods.left) ||
                           (mods.right >= 0 && kw0 + 31 - i0 - diag > mods.right);
        const float slope_l2 = slope * kLog2e;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int fd = i0 + 4 * g + diag - (kw0 + 16 * kb + c);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse_t + 16 * qb + 4 * g);
            const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dlt_t + 16 * qb + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float d = (float)fd + (float)(16 * qb + r);  // exact in fp32
              const float nl = l4[r] * -kLog2e;
              const float base = kAlibi ? __builtin_fmaf(-slope_l2, __builtin_fabsf(d), nl) : nl;
              float p, gd = 1.f;
              if constexpr (kCap) {
                const float th = __builtin_fmaf(
                    -2.f, __builtin_amdgcn_rcpf(exp2_fast(sc[qb][kb][r] * cap_in) + 1.f), 1.f);
                gd = __builtin_fmaf(-th, th, 1.f);
                p = exp2_fast(__builtin_fmaf(th, cap_l2, base));
              } else {
                p = exp2_fast(__builtin_fmaf(sc[qb][kb][r], sigma_l2, base));
              }
              sc[qb][kb][r] = p;
              const float tv = p * (dp[qb][kb][r] - d4[r]);
              dp[qb][kb][r] = kCap ? tv * gd : tv;
            }
          }
          if (mmask) {
            // Row offset o = 16 qb + r is visible iff fd + o lies in
            // [lo_i, hi_i[kb]] (selects, as in the dQ kernel).
            const int o_lo = lo_i - fd, o_hi = hi_i[kb] - fd;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int o = 16 * qb + r;
                const bool vis = o >= o_lo && o <= o_hi;
                sc[qb][kb][r] = vis ? sc[qb][kb][r] : 0.f;
                dp[qb][kb][r] = vis ? dp[qb][kb][r] : 0.f;
              }
            }
          }
          pack_kb(kb);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse_t + 16 * qb + 4 * g);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dlt_t + 16 * qb + 4 * g);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = exp2_fast(__builtin_fmaf(sc[qb][kb][r], c_log2, -l4[r] * kLog2e));
              sc[qb][kb][r] = p;
              dp[qb][kb][r] = p * (dp[qb][kb][r] - d4[r]);
            }
          }
        }
        if (need_mask) {
          // Row i = i0 + 4 g + o, o = 16 qb + r, is visible to key j iff
          // i < Nq and (causal) j <= i + diag: o in [o_lo[kb], o_hi[kb]].
          // Selects, so that an infinite P of a hidden pair goes away.
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int j = kw0 + 16 * kb + c;
            const int o_lo = CAUSAL ? j - diag - i0 - 4 * g : -(1 << 30);
            const int o_hi = j < Nk ? Nq - i0 - 4 * g - 1 : -(1 << 30) - 1;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int o = 16 * qb + r;
                const bool vis = o >= o_lo && o <= o_hi;
                sc[qb][kb][r] = vis ? sc[qb][kb][r] : 0.f;
                dp[qb][kb][r] = vis ? dp[qb][kb][r] : 0.f;
              }
            }
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pack_kb(kb);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x2_t a0 = lds_read_tr4(dt + t_rd + 16 * db);
        const u32x2_t a1 = lds_read_tr4(dt + t_rd + 16 * RS + 16 * db);
        const u32x4_t av = {a0[0], a0[1], a1[0], a1[1]};
        const u32x2_t b0 = lds_read_tr4(qt + t_rd + 16 * db);
        const u32x2_t b1 = lds_read_tr4(qt + t_rd + 16 * RS + 16 * db);
        const u32x4_t aq = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dv[db][kb] = mfma_16x16x32<BF16>(av, pb[kb], dv[db][kb]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dk[db][kb] = mfma_16x16x32<BF16>(aq, sb[kb], dk[db][kb]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // dK = scale * dK^T, dV = dV^T, rounded; keys >= Nk fall outside the range.
  const rsrc_t dkr = make_rsrc(dK + kv_off, kspan);
  const rsrc_t dvr = make_rsrc(dV + kv_off, kspan);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int ovoff = (int)((16 * kb + c) * kv_rs * 2) + 8 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      buf_store8(pack4<BF16>(dk[db][kb] * scale), dkr, ovoff + 32 * db);
      buf_store8(pack4<BF16>(dv[db][kb]), dvr, ovoff + 32 * db);
    }
  }
}

}  // namespace eta
