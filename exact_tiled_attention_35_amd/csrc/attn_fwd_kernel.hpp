// Exact tiled attention forward for gfx950 (MI355X, CDNA4).
//
// The computation is exact softmax attention, softmax(Q K^T * scale) V, per
// (batch, query head) -- the formula of the interface section of the page
// "FlashAttention: exakte Attention-Kernel fuer CUDA und ROCm" (hysenlabs.com).
// It follows the five-stage map of unite.ai's "Was ist FlashAttention?"
// (section "Eine fuenfstufige Betriebsuebersicht"): Q, K, V are cut into tiles
// (stage 1), small K/V blocks go to fast on-chip memory, here LDS (stage 2),
// local scores and a running normalisation are computed (stage 3), outputs are
// accumulated without ever materialising the full score matrix (stage 4), and
// the work is laid out for the target accelerator (stage 5).  The dense score
// matrix that tokenwerk.de's "FlashAttention" page sizes (section "Warum
// Kacheln beim Speicherzugriff helfen": 2 MiB per head at N = 1,024, 32 MiB at
// N = 4,096) never leaves registers.
//
// gfx950 mapping (our own design, not from the pages):
//  * One workgroup = 4 wave64s = one block of 128 query rows of one (b, head);
//    each wave owns 32 query rows.
//  * Both products run transposed on v_mfma_f32_32x32x16_{bf16,f16}:
//        S^T = K . Q^T   (A = K tile from LDS, B = Q^T kept in VGPRs, or at
//                         d = 256 read from an LDS copy of the Q tile)
//        O^T = V^T . P^T (A = V^T tile from LDS, B = P^T straight from the
//                         S^T accumulators)
//    With the 32x32 accumulator layout (lane l, register r holds row
//    8*(r/4) + 4*(l/32) + r%4, column l%32), column = query, so every lane owns
//    ONE query row: the running max / sum / rescale factor are per-lane
//    scalars and a row reduction is an in-lane reduction plus one exchange
//    between lanes l and l+32.
//  * K and V tiles are copied HBM -> LDS by direct buffer loads (no register
//    staging), row-major with padded rows that make every operand read
//    bank-conflict free; V reaches the MFMA as V^T through the LDS transpose
//    read ds_read_b64_tr_b16.  Two stages: the loads of tile t+1 are in
//    flight while tile t is computed, one barrier per tile.
//  * Online softmax in the log2 domain: t = s * scale * log2(e), p = 2^(t - m).
//    The running maximum m is only raised when a tile's maximum exceeds it
//    by more than kRescaleThreshold (p then stays <= 2^threshold).  Because
//    the same m is used for the sum l and for O, the result is still exact;
//    the rescale of O is skipped on almost every tile.  Tiles every row sees
//    completely skip the tile maximum altogether ("lean" tiles, below).
//  * Causal: tiles entirely above the diagonal are never loaded; tiles that
//    cross it (and ragged tails) are masked per element.  On those tiles P is
//    fed to the PV product as hi + lo halves (two MFMAs), which keeps the
//    early causal rows -- where one P entry carries most of the weight -- at
//    the accuracy of the output rounding.
//  * The row sum l is accumulated from the unrounded fp32 p.
//  * Epilogue: O /= l, rounded to nearest-even, staged through LDS so that
//    each store writes 16 contiguous bytes per lane; lse = (m + log2 l) * ln 2.
//  * Template switches: MODS adds the score variants (sliding window, ALiBi,
//    softcap), VARLEN takes the rows of packed variable-length sequences
//    from prefix sums, SPARSE visits only the key blocks a block mask flags;
//    with all off the kernel is the plain one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gfx950_ops.hpp"

namespace eta {

constexpr float kLog2e_f = 1.44269504088896340736f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p <= 256 between rescales
// Unmasked tiles keep the current running max unless a row's tile sum
// exceeds this (every p then stays far inside the fp16 range of P).
constexpr float kSumLimit = 32768.0f;

// Epilogue of a wave's 32 query rows: O^T accumulators (lane l holds
// 4-element pieces of row l % 32) are scaled by inv, rounded to the element
// type and stored.  The wave stages its rounded rows in its own slice of LDS
// (row stride D + 8 elements, 16-byte aligned rows) and reads them back 16
// contiguous bytes per lane, so that each store instruction writes whole row
// segments (64 / (D / 8) rows x D elements) instead of 16 bytes of 32 rows.
// Rows 16-31 swap the two 8-byte halves of each 16-byte chunk (the reads
// swap them back), which spreads a write's 32 rows over all 64 banks if a
// pass serves 32 lanes; the counters still show 96 bank-conflict cycles per
// wave in this staging at d = 128 (none in the tile loops), about 1 % of the
// LDS's busy cycles, once per workgroup.  The caller guarantees that no wave
// still reads the LDS area (4 x 32 x (D + 8) elements from smem).  Stores of
// rows past the descriptor's range (rows >= Nq) are dropped.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows(uint16_t* smem, int wave, int lane,
                                           const f32x16_t (&oacc)[D / 32], float inv, rsrc_t orr,
                                           int64_t q_rs) {
  constexpr int ORS = D + 8;
  const int l32 = lane & 31, hh = lane >> 5;
  uint16_t* const ost = smem + wave * 32 * ORS;
  const int half = 4 * (hh ^ (l32 >> 4));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4_t o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * inv;
      *reinterpret_cast<u32x2_t*>(ost + l32 * ORS + 32 * db + 8 * g + half) = pack4<BF16>(o4);
    }
  }
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + rr;
    u32x4_t v16 = *reinterpret_cast<const u32x4_t*>(ost + row * ORS + 8 * cc);
    if (row >= 16) v16 = u32x4_t{v16[2], v16[3], v16[0], v16[1]};
    buf_store16(v16, orr, (int)(row * q_rs * 2) + 16 * cc);
  }
}

// Tile shape per head dimension.
//
// LDS holds two stages; each stage has a K region and a V region, both
// row-major [BN keys][D] with padded rows.  gfx950's LDS has 64 banks of 4
// bytes (256 bytes per clock, measured).  A ds_read_b128 pass serves 16 lanes
// (16 rows here), so the K row stride is an odd multiple of 4 dwords; a
// ds_read_b64_tr_b16 pass serves 32 lanes (4 rows x 64 bytes here), so the V
// row stride is an odd multiple of 16 dwords.  Both make the operand reads
// bank-conflict free.  Tiles are filled by direct global->LDS buffer loads,
// 64 lanes x 16 bytes per instruction, one 16-byte "slot" per lane; pad slots
// receive a duplicate chunk that is never read.
template <int D>
struct TileCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;                 // query rows per workgroup
  static constexpr int BN = (D >= 256) ? 32 : 64;        // keys per K/V tile
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int KCP = kChunks + 1;                // K row, in 16-byte slots
  static constexpr int VCP = kChunks + 4;                // V row, in 16-byte slots
  static constexpr int KS = 8 * KCP;                     // K row stride (elements)
  static constexpr int VS = 8 * VCP;                     // V row stride (elements)
  static constexpr int kKInst = (BN * KCP + 63) / 64;    // direct-load instructions per K tile
  static constexpr int kVInst = (BN * VCP + 63) / 64;    // ... per V tile
  static constexpr int kKElems = kKInst * 64 * 8;        // K region (elements)
  static constexpr int kVElems = kVInst * 64 * 8;        // V region (elements)
  static constexpr int kStage = kKElems + kVElems;       // one stage (elements)
  static constexpr int kKInstPerWave = (kKInst + kWaves - 1) / kWaves;
  static constexpr int kVInstPerWave = (kVInst + kWaves - 1) / kWaves;
  // d = 256: the Q tile lives in LDS (read as the B operand like K), so that
  // the 128 O accumulators fit in architectural VGPRs next to S and P.
  static constexpr bool kQInLds = (D >= 256);
  static constexpr int kQInst = (BM * KCP + 63) / 64;     // direct-load instructions for Q
  static constexpr int kQInstPerWave = (kQInst + kWaves - 1) / kWaves;
  static constexpr int kQElems = kQInLds ? kQInst * 64 * 8 : 0;
  static constexpr int kLdsElems = 2 * kStage + kQElems;
  static constexpr int kMinWavesPerEU = (D >= 256) ? 1 : 2;
  // Unmasked tiles after the first skip the tile maximum (see the kernel).
  static constexpr bool kLeanTiles = true;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile sizes must be multiples of 32");
  static_assert((KS / 2) % 8 == 4 && (VS / 2) % 32 == 16, "bank-conflict-free strides");
};


template <int D, bool BF16, bool CAUSAL, bool MODS = false, bool VARLEN = false, bool SPARSE = false>
__global__ void __launch_bounds__(TileCfg<D>::kThreads, TileCfg<D>::kMinWavesPerEU)
attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb,
                int total, float c_log2, int prescale, ScoreMods mods, VarlenArgs va,
                BlockMaskArgs bm) {
  using C = TileCfg<D>;
  static_assert(!(SPARSE && (MODS || VARLEN)), "block sparsity is an instance of its own");
  static_assert(kMaskBlock % C::BN == 0 && kMaskBlock == C::BM, "a mask block is whole tiles");
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NKS = D / 16;  // k-steps of the S^T product
  constexpr int NKB = BN / 32; // 32-key blocks per tile
  constexpr int NDB = D / 32;  // 32-column blocks of O^T
  constexpr int NKK = BN / 16; // 16-key steps of the PV product
  constexpr int KCPR = D / 8;  // 16-byte chunks per row

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const WorkItem w = VARLEN ? map_workgroup_packed(blockIdx.x, nqb, Hq, va.pairs)
                           : map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;

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
  // Row qw0 of (b, hq) in q / out; row 0 of (b, hkv) in k / v.
  const int64_t qo_off = (q_row0 + qw0) * q_rs + (int64_t)w.hq * D;
  const uint16_t* Kh = K + (k_row0 * Hkv + hkv) * D;
  const uint16_t* Vh = V + (k_row0 * Hkv + hkv) * D;

  // ---- Q (B operand of S^T = K Q^T): fragments resident in VGPRs for the
  // whole loop, or (d = 256) the workgroup's Q tile in LDS.  Rows past Nq
  // read as zero (outside the descriptor's range).
  u32x4_t qf[C::kQInLds ? 1 : NKS];
  uint16_t* const qs = smem + 2 * C::kStage;
  if constexpr (!C::kQInLds) {
    const rsrc_t qr = make_rsrc(Q + qo_off, span_bytes(qw0, 32, Nq, q_rs, D));
    const int voff = (int)(l32 * q_rs * 2) + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qr, voff + 32 * ks);
  } else {
    const int64_t q0_off = (q_row0 + q0) * q_rs + (int64_t)w.hq * D;
    const rsrc_t qr = make_rsrc(Q + q0_off, span_bytes(q0, BM, Nq, q_rs, D));
#pragma unroll
    for (int i = 0; i < C::kQInstPerWave; ++i) {
      const int j = wave + C::kWaves * i;
      const int sl = 64 * j + lane;
      const int row = min(sl / C::KCP, BM - 1), c = min(sl % C::KCP, C::kChunks - 1);
      if (j < C::kQInst) buf_load_lds16(qr, qs + 512 * j, (int)(row * q_rs * 2) + 16 * c);
    }
  }
  const int q_rd = (wave * 32 + l32) * KS + 8 * hh;  // this lane's Q row in LDS

  // ---- Key range of the workgroup and of this wave.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);
  // Window: keys right of the last row's window are never loaded, tiles left
  // of the first row's window are skipped (jb = first tile), and a wave skips
  // tiles outside its own rows' windows.
  int jb = 0, w_begin = 0;
  if constexpr (MODS) {
    if (mods.right >= 0) {
      kv_end = min(kv_end, max(0, min(q0 + BM, Nq) + diag + mods.right));
      if (rows_end > qw0) w_end = min(w_end, max(0, rows_end + diag + mods.right));
    }
    if (mods.left >= 0) {
      jb = max(0, q0 + diag - mods.left) / BN;
      w_begin = qw0 + diag - mods.left;
    }
  }
  int nt = kv_end > jb * BN ? (kv_end - jb * BN + BN - 1) / BN : 0;

  // ---- Block sparsity: the tiles of flagged key blocks below kv_end, in key
  // order.  Each wave reads the flags of 64 key blocks per step (one byte per
  // lane, a ballot makes them wave-uniform), counts the tiles it will visit
  // (nt) and those every row sees whole (sp_nf, the lean/full bodies), and
  // then walks the flagged blocks; unflagged tiles are never loaded.
  constexpr int TPB = kMaskBlock / BN;  // tiles per mask block
  int sp_nf = 0, sp_chunk = 0, sp_blk = 0, sp_sub = TPB, sp_cur = 0, sp_nchunks = 0;
  uint64_t sp_bits = 0;
  const int nkb_eff = (kv_end + kMaskBlock - 1) / kMaskBlock;
  const int64_t sp_row = ((int64_t)w.b * bm.heads + (bm.heads == 1 ? 0 : w.hq)) * nqb + w.qblk;
  // this row of flags; flags past kv_end read as 0 (unused without SPARSE)
  const rsrc_t sp_mr = make_rsrc(SPARSE ? bm.mask + sp_row * bm.nkb : nullptr, SPARSE ? nkb_eff : 0);
  if constexpr (SPARSE) {
    sp_nchunks = (nkb_eff + 63) / 64;
    int nf_plain = Nk / BN;
    if (CAUSAL) nf_plain = min(nf_plain, max(0, (q0 + diag + 1) / BN));
    const int full_blocks = nf_plain / TPB, full_rem = nf_plain % TPB;
    const int last = nkb_eff - 1;  // may hold fewer than TPB tiles
    const int last_tiles = (kv_end - kMaskBlock * last + BN - 1) / BN;
    int blocks = 0, nf_blocks = 0;
    nt = 0;
    for (int c = 0; c < sp_nchunks; ++c) {
      const uint64_t bits = flag_word(sp_mr, c, 1, lane);
      if (c == 0) sp_bits = bits;
      blocks += __builtin_popcountll(bits);
      const int below = full_blocks - 64 * c;  // blocks of this chunk under full_blocks
      nf_blocks += __builtin_popcountll(below >= 64 ? bits : below <= 0 ? 0ull
                                        : bits & ((1ull << below) - 1));
      if (full_rem && below >= 0 && below < 64 && ((bits >> below) & 1)) sp_nf += full_rem;
      if (last / 64 == c && ((bits >> (last % 64)) & 1)) nt -= TPB - last_tiles;
    }
    nt += TPB * blocks;
    sp_nf += TPB * nf_blocks;
  }
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

  // ---- Direct global->LDS tile loads.  This wave issues the K (V) tile's
  // instructions j = wave, wave + 4, ...; lane -> 16-byte slot 64 j + lane ->
  // (row, chunk) of the padded layout; offsets are loop-invariant.
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

  // ---- Operand reads from LDS (loop-invariant parts of the element offsets).
  const int g16 = lane >> 4, i16 = lane & 15;
  const int k_rd = l32 * KS + 8 * hh;
  const int v_rd = C::kKElems + (4 * hh + (i16 >> 2)) * VS + 16 * (g16 & 1) + 4 * (i16 & 3);

  // ---- Running state (per lane = per query row).
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY;  // running max of t = s * c_log2 (log2 units)
  float lsum = 0.f;     // this lane half's share of the running sum
  // A window alone leaves the scores as they are ("plain"); softcap or ALiBi
  // transform them, and the transformed scores are held in log2 units.
  const bool plain = !MODS || (!mods.slopes && !(mods.cap > 0.f));
  const float ce = (!plain || prescale) ? 1.0f : c_log2;
  float slope = 0.f;
  if constexpr (MODS) slope = mods.slopes ? mods.slopes[w.hq] : 0.f;
  const bool alibi_only = MODS && mods.slopes && !(mods.cap > 0.f) && mods.left < 0 && mods.right < 0;
  const float slope_l2 = slope * kLog2e_f, sigma_l2 = mods.sigma * kLog2e_f;
  const bool cap_only = MODS && !mods.slopes && mods.cap > 0.f && mods.left < 0 && mods.right < 0;
  // softcap: exp2 argument 2 x log2e with x = s sigma / cap; output scale cap log2e
  const float cap_in = cap_only ? mods.sigma * __builtin_amdgcn_rcpf(mods.cap) * 2.88539008177792681472f : 0.f;
  const float cap_l2 = mods.cap * kLog2e_f;

  if constexpr (SPARSE) {
    if (nt > 0) sp_cur = sparse_next();
  }
  if (nt > 0) issue_tile(SPARSE ? sp_cur : jb * BN, smem);
  __builtin_amdgcn_s_waitcnt(0);  // Q fragments and tile 0 have landed
  __syncthreads();

  // S^T = K Q^T for BN keys x 32 queries, from the K tile at `st`.
  auto compute_s = [&](const uint16_t* st, f32x16_t (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(st + k_rd + kb * 32 * KS + 16 * ks);
        u32x4_t b;
        if constexpr (C::kQInLds)
          b = *reinterpret_cast<const u32x4_t*>(qs + q_rd + 16 * ks);
        else
          b = qf[ks];
        s[kb] = mfma_32x32x16<BF16>(a, b, s[kb]);
      }
    }
    if constexpr (C::kQInLds) {
      // d = 256 runs one wave per SIMD, so no other wave covers the LDS
      // latency: the Q and K operand reads are kept three k-steps ahead of
      // the MFMAs (deeper was measured slower)
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < NKS - 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    if (prescale) {  // scale <= 0: take the max of s*c directly
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] *= c_log2;
    }
  };

  // Tile row maximum (in-lane, then across the two lane halves); m is raised
  // when the tile max exceeds it by more than `threshold`, and what was
  // accumulated is rescaled.
  auto raise_max = [&](const f32x16_t (&s)[NKB], float threshold) {
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = max3(tmax, s[kb][r], s[kb][r + 1]);
    }
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
    const float tm = tmax * ce;
    if (tm > m + threshold) {
      const float alpha = exp2_fast(m - tm);
      m = tm;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
  };

  // p = 2^(s*c - m) in place; returns this lane half's sum of the unrounded p.
  auto exponentiate = [&](f32x16_t (&s)[NKB], auto m_finite) {
    const float mb = (decltype(m_finite)::value || m != -INFINITY) ? m : 0.f;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(s[kb][r], ce, -mb));
        const float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], ce, -mb));
        s[kb][r] = p0;
        s[kb][r + 1] = p1;
        ps0 += p0;
        ps1 += p1;
      }
    }
    return ps0 + ps1;
  };

  // Tile t.  Mode kLean: every key visible to every row and m already
  // finite -- the scores are exponentiated against the current m without a
  // tile maximum; a partial row sum above kSumLimit (a score far above m,
  // rare) sends the wave through the maximum path for this tile, recomputing S
  // from the K tile still in LDS.  Mode kFull: every key visible, tile
  // maximum first.  Mode kMasked: tile maximum first, per-element masking
  // where the tile crosses the causal diagonal or the ragged end.  The same m
  // enters the row sum and O in every case, so both are exact.
  constexpr int kLean = 0, kFull = 1, kMasked = 2;
  auto tile = [&](int t, auto mode) {
    constexpr int kMode = decltype(mode)::value;
    const int j0 = SPARSE ? sp_cur : (jb + t) * BN;
    // Tile t+1 streams into the other stage while this one is computed (that
    // stage was last read in iteration t-1, before the barrier that ended it).
    if (t + 1 < nt) {
      int jn = j0 + BN;
      if constexpr (SPARSE) jn = sp_cur = sparse_next();
      issue_tile(jn, smem + ((t + 1) & 1) * C::kStage);
    }
    const uint16_t* st = smem + (t & 1) * C::kStage;

    // wave-uniform: skip tiles above this wave's diagonal (or outside its window)
    if (j0 < w_end && (!MODS || j0 + BN > w_begin)) {
      f32x16_t s[NKB];
      // The matrix phases (S^T here, O^T below) run at raised wave priority,
      // so that on a SIMD shared with a wave in its softmax phase the MFMA
      // issues first and that wave's VALU work fills the remaining slots.
      __builtin_amdgcn_s_setprio(1);
      compute_s(st, s);
      __builtin_amdgcn_s_setprio(0);
      bool need_mask = false;
      float psum;
      if constexpr (kMode == kLean) {
        psum = exponentiate(s, std::true_type{});
        if (__builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) != 0) {
          compute_s(st, s);
          raise_max(s, 0.0f);
          psum = exponentiate(s, std::true_type{});
        }
      } else {
        // Mask keys past the end and (causal) above the diagonal.
        need_mask = kMode == kMasked &&
                    ((j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag));
        if constexpr (MODS) {
          // Softcap, ALiBi and the window on every element; log2 units.
          if (mods.left >= 0 && j0 < qw0 + 31 + diag - mods.left) need_mask = true;
          if (mods.right >= 0 && j0 + BN - 1 > qw0 + diag + mods.right) need_mask = true;
          // Fast paths for tiles every key of which every row sees (no
          // masking): softcap alone, and ALiBi alone on a tile whose keys all
          // lie on one side of every row's diagonal key (the distance keeps
          // its sign, so the bias is linear in the key offset: two FMAs per
          // score).  Other tiles take the general per-element transform.
          const bool below = j0 + BN - 1 <= qw0 + diag;
          const bool above = !CAUSAL && j0 >= qw0 + 31 + diag;
          if (cap_only && (!CAUSAL || below) && j0 + BN <= Nk) {
            // t = cap * tanh(s * sigma / cap) * log2e, tanh(x) = 1 - 2 / (e^(2x) + 1)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float e = exp2_fast(s[kb][r] * cap_in);
                s[kb][r] = __builtin_fmaf(-2.0f * cap_l2, __builtin_amdgcn_rcpf(e + 1.0f), cap_l2);
              }
            }
          } else if (alibi_only && (below || above) && j0 + BN <= Nk) {
            // t = s*sigma*log2e - slope*log2e*|my_q + diag - j|, with
            // j = j0 + kb*32 + 8*(r/4) + 4*hh + r%4
            const float ss = below ? slope_l2 : -slope_l2;
            const float lane_base = -ss * (float)(my_q + diag - j0 - 4 * hh);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float off = (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
                s[kb][r] = __builtin_fmaf(s[kb][r], sigma_l2, __builtin_fmaf(ss, off, lane_base));
              }
            }
          } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const int dist = my_q + diag - j;
                float tv = s[kb][r];
                if (!plain) {
                  tv *= mods.sigma;
                  if (mods.cap > 0.f) tv = mods.cap * tanh_fast(tv * __builtin_amdgcn_rcpf(mods.cap));
                  tv = (tv - slope * (float)(dist < 0 ? -dist : dist)) * kLog2e_f;
                }
                const bool vis = j < Nk && (!CAUSAL || dist >= 0) &&
                                 (mods.left < 0 || dist <= mods.left) &&
                                 (mods.right < 0 || -dist <= mods.right);
                s[kb][r] = vis ? tv : -INFINITY;
              }
            }
          }
        } else if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
              const bool vis = j < Nk && (!CAUSAL || j <= my_q + diag);
              s[kb][r] = vis ? s[kb][r] : -INFINITY;
            }
          }
        }
        raise_max(s, kRescaleThreshold);
        psum = exponentiate(s, std::false_type{});
      }
      lsum += psum;

      // O^T += V^T P^T.  PV step kk covers keys 16kk..16kk+15; lane half hh
      // feeds keys {4hh..4hh+3, 8+4hh..8+4hh+3}, which registers
      // 8*(kk%2)..+7 of S^T block kk/2 hold.  The A operand (V^T, 8 keys at
      // one column) comes from two LDS transpose reads of row-major V.
      // Causal tiles that cross the diagonal feed P as hi + lo halves (two
      // MFMAs per step); the choice is made once per tile, not per MFMA.
      auto pv_product = [&](auto with_lo) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int kb = kk >> 1, r0 = 8 * (kk & 1);
          f32x8_t pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = s[kb][r0 + e];
          const u32x4_t phi = pack8<BF16>(pv);
          u32x4_t plo;
          if constexpr (decltype(with_lo)::value) plo = pack8<BF16>(pv - unpack8<BF16>(phi));
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x2_t x0 = lds_read_tr4(st + v_rd + 16 * kk * VS + 32 * db);
            const u32x2_t x1 = lds_read_tr4(st + v_rd + (16 * kk + 8) * VS + 32 * db);
            const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
            oacc[db] = mfma_32x32x16<BF16>(a, phi, oacc[db]);
            if constexpr (decltype(with_lo)::value) oacc[db] = mfma_32x32x16<BF16>(a, plo, oacc[db]);
          }
        }
        if constexpr (C::kQInLds && !decltype(with_lo)::value) {
          // and the V^T operand reads four MFMAs ahead
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int i = 0; i < NKK * NDB - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
      };
      // P as hi + lo keeps rows that see few keys, where one P entry carries
      // most of the weight, at the output's rounding (with a block mask a row
      // may keep only the keys of a ragged last block).  A tile masked only by
      // the left edge of a window of at least 128 keys needs no lo half:
      // every row it holds sees at least that many keys.
      bool with_lo = (CAUSAL || MODS || SPARSE) && need_mask;
      if constexpr (MODS) {
        const bool right_edge = (CAUSAL && j0 + BN - 1 > qw0 + diag) ||
                                (mods.right >= 0 && j0 + BN - 1 > qw0 + diag + mods.right);
        if (plain && mods.left >= 127 && !right_edge && j0 + BN <= Nk) with_lo = false;
      }
      __builtin_amdgcn_s_setprio(1);
      if (with_lo)
        pv_product(std::true_type{});
      else
        pv_product(std::false_type{});
      __builtin_amdgcn_s_setprio(0);
    }

    __builtin_amdgcn_s_waitcnt(0);  // tile t+1 has landed in LDS
    __syncthreads();
  };
  // Tiles before nf are visible to every row of the workgroup: the first of
  // them (m still -inf) takes the full body, the rest the lean one; tiles
  // from nf on take the masked body.  Separate loops keep each body's
  // register allocation free of the others' state.
  // Tiles [t_lo, nf) are visible to every row of the workgroup.  A window
  // adds masked tiles at its left edge (before t_lo) and bounds nf on the
  // right; softcap and ALiBi change every score, so with them every tile
  // takes the masked body.
  int nf = Nk / BN;
  if (CAUSAL) nf = min(nf, max(0, (q0 + diag + 1) / BN));
  int t_lo = 0;
  if constexpr (MODS) {
    if (mods.right >= 0) nf = min(nf, max(0, (q0 + diag + mods.right + 1) / BN));
    if (mods.left >= 0) {
      const int q_last = min(q0 + BM, Nq) - 1;
      t_lo = max(0, (q_last + diag - mods.left + BN - 1) / BN - jb);
    }
    nf -= jb;
    if (!plain) t_lo = nf = 0;
  }
  if constexpr (SPARSE) nf = sp_nf;
  nf = min(max(nf, 0), nt);
  t_lo = min(t_lo, nf);
  using LeanMode = std::integral_constant<int, kLean>;
  using FullMode = std::integral_constant<int, kFull>;
  using MaskedMode = std::integral_constant<int, kMasked>;
  int t = 0;
  if constexpr (MODS) {
    for (; t < t_lo; ++t) tile(t, MaskedMode{});
  }
  if constexpr (C::kLeanTiles) {
    if (t < nf) tile(t++, FullMode{});
    for (; t < nf; ++t) tile(t, LeanMode{});
  } else {
    for (; t < nf; ++t) tile(t, FullMode{});
  }
  for (; t < nt; ++t) tile(t, MaskedMode{});

  // ---- Epilogue: normalise, round, store O and the logsumexp (every wave
  // passed the last tile's barrier: no wave reads the stages any more).
  static_assert(C::kWaves * 32 * (D + 8) <= C::kLdsElems, "the staged rows fit the stages");
  const float lt = lsum + __shfl_xor(lsum, 32);
  store_rows<D, BF16>(smem, wave, lane, oacc, lt > 0.f ? 1.0f / lt : 0.f,
                      make_rsrc(O + qo_off, span_bytes(qw0, 32, Nq, q_rs, D)), q_rs);
  const int nrows = max(0, min(32, Nq - qw0));
  const rsrc_t lr = make_rsrc(LSE + lse_off + qw0, nrows * 4);
  buf_store4(lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY, lr, 4 * l32);
}

}  // namespace eta
