// Exact tiled attention forward for grids smaller than the GPU (gfx950).
//
// The same computation as attn_fwd_kernel (exact softmax attention with an
// online softmax, tile by tile; the formula of the interface section of the
// page "FlashAttention: exakte Attention-Kernel fuer CUDA und ROCm",
// hysenlabs.com), laid out for problems whose (batch, head, 128-row block)
// count leaves most of the 256 compute units idle -- a single head of 1,024
// rows has 8 such blocks.  Each workgroup takes 32 query rows and its four
// waves split the keys between them: wave w streams its own quarter of the
// key tiles through its own two LDS stages (no workgroup barrier in the
// loop), keeps its own running maximum m_w, row sum l_w and unnormalised
// output O_w, and the four partial results are merged through LDS at the
// end:
//     M = max_w m_w,  L = sum_w l_w 2^(m_w - M),  O = sum_w O_w 2^(m_w - M) / L,
// lse = (M + log2 L) ln 2 -- the logsumexp merge that also combines the key
// splits of the KV-cache decode.  The version history on the hysenlabs.com
// page (section "Von 2.0 bis 2.7", version 2.2) names this kind of key
// splitting for short-query inference.  The merge runs in a fixed order, so
// the result is bitwise reproducible.
//
// Per wave the tile body is the one of attn_fwd_kernel: S^T = K Q^T and
// O^T = V^T P^T on v_mfma_f32_32x32x16 (one lane per query row), exp2 in the
// log2 domain with a lazily raised maximum (no tile maximum at all on tiles
// after the wave's first that every row sees whole), row sums from the unrounded p,
// causal and ragged masking per element, P as hi + lo halves on tiles that
// cross the causal diagonal (and on every tile of a block whose first row
// sees fewer than 128 keys).  Tiles are 32 keys, so that each wave's stages
// fit in LDS: three at d = 64 (loads two tiles ahead), two at d = 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.hpp"

namespace eta {

template <int D>
struct SplitCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32;                          // query rows per workgroup
  static constexpr int BN = 32;                          // keys per tile
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int KCP = kChunks + 1;                // K row, in 16-byte slots
  static constexpr int VCP = kChunks + 4;                // V row, in 16-byte slots
  static constexpr int KS = 8 * KCP, VS = 8 * VCP;       // row strides (elements)
  static constexpr int kKInst = (BN * KCP + 63) / 64;    // direct-load instructions per K tile
  static constexpr int kVInst = (BN * VCP + 63) / 64;    // ... per V tile
  static constexpr int kKElems = kKInst * 64 * 8;
  static constexpr int kVElems = kVInst * 64 * 8;
  static constexpr int kStage = kKElems + kVElems;       // one stage (elements)
  // Stages per wave: three at d = 64 (loads run two tiles ahead), two at
  // d = 128 (three would not fit the 160 KiB of LDS).
  static constexpr int kStages = (D == 64) ? 3 : 2;
  static constexpr int kWaveElems = kStages * kStage;    // a wave's stages
  static constexpr int kTileInst = kKInst + kVInst;      // load instructions per tile
  // merge area (fp32, reusing the stages): O_w in accumulator order, m_w, l_w
  static constexpr int kMergeFloats = kWaves * BM * D + 2 * kWaves * 64;
  static constexpr int kLdsElems =
      (kWaves * kWaveElems > 2 * kMergeFloats) ? kWaves * kWaveElems : 2 * kMergeFloats;
  static_assert(D == 64 || D == 128, "the key-split kernel serves d = 64 and d = 128");
  static_assert((KS / 2) % 8 == 4 && (VS / 2) % 32 == 16, "bank-conflict-free strides");
};

template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(SplitCfg<D>::kThreads, 1)
attn_fwd_splitk_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                       const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                       float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb,
                       float c_log2, int prescale) {
  using C = SplitCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NKS = D / 16;  // k-steps of the S^T product
  constexpr int NDB = D / 32;  // 32-column blocks of O^T
  constexpr int NKK = BN / 16; // 16-key steps of the PV product
  constexpr float kRescale = 8.0f;      // log2 units: p <= 256 between rescales
  constexpr float kSumLimit = 32768.0f;  // lean tiles: partial row sums above this retake the max

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // blockIdx -> (b, head, 32-row block); the blocks of a head are adjacent
  const int qblk = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const int q0 = qblk * BM;
  const int my_q = q0 + l32;
  const int diag = Nk - Nq;

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const int64_t qo_off = ((int64_t)b * Nq + q0) * q_rs + (int64_t)hq * D;
  const uint16_t* Kh = K + ((int64_t)b * Nk * Hkv + hkv) * D;
  const uint16_t* Vh = V + ((int64_t)b * Nk * Hkv + hkv) * D;

  // Q^T fragments (B operand), rows past Nq read as zero.
  u32x4_t qf[NKS];
  {
    const rsrc_t qr = make_rsrc(Q + qo_off, span_bytes(q0, BM, Nq, q_rs, D));
    const int voff = (int)(l32 * q_rs * 2) + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qr, voff + 32 * ks);
  }

  // Keys of the workgroup, in whole tiles, and this wave's quarter of them.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int nt_all = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int per_wave = (nt_all + C::kWaves - 1) / C::kWaves;
  const int t_begin = min(nt_all, wave * per_wave);
  const int nt = min(nt_all, t_begin + per_wave) - t_begin;

  // This wave's direct global->LDS loads: all instructions of its tiles.
  uint16_t* const wst = smem + wave * C::kWaveElems;
  int koff[C::kKInst], voff[C::kVInst];
#pragma unroll
  for (int j = 0; j < C::kKInst; ++j) {
    const int sl = 64 * j + lane;
    koff[j] = (int)(min(sl / C::KCP, BN - 1) * kv_rs * 2) + 16 * min(sl % C::KCP, C::kChunks - 1);
  }
#pragma unroll
  for (int j = 0; j < C::kVInst; ++j) {
    const int sl = 64 * j + lane;
    voff[j] = (int)(min(sl / C::VCP, BN - 1) * kv_rs * 2) + 16 * min(sl % C::VCP, C::kChunks - 1);
  }
  auto issue_tile = [&](int j0, uint16_t* stage) {
    const int bytes = span_bytes(j0, BN, Nk, kv_rs, D);
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, bytes);
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, bytes);
#pragma unroll
    for (int j = 0; j < C::kKInst; ++j) buf_load_lds16(kr, stage + 512 * j, koff[j]);
#pragma unroll
    for (int j = 0; j < C::kVInst; ++j) buf_load_lds16(vr, stage + C::kKElems + 512 * j, voff[j]);
  };
  const int k_rd = l32 * KS + 8 * hh;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_rd = C::kKElems + (4 * hh + (i16 >> 2)) * VS + 16 * (g16 & 1) + 4 * (i16 & 3);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY;  // running max of s * c_log2 (log2 units)
  float lsum = 0.f;     // this lane half's share of the running sum
  const float ce = prescale ? 1.0f : c_log2;

  // s_waitcnt immediate (GFX9 encoding) that waits until at most n vector
  // memory operations are outstanding and leaves the other counters alone.
  auto wait_vm = [](auto n) {
    constexpr int v = decltype(n)::value;
    __builtin_amdgcn_s_waitcnt((v & 15) | (7 << 4) | (15 << 8) | ((v >> 4) << 14));
  };
  constexpr int AHEAD = C::kStages - 1;  // tiles in flight beyond the current one
  if (nt > 0) issue_tile(t_begin * BN, wst);
  if (AHEAD > 1 && nt > 1) issue_tile((t_begin + 1) * BN, wst + C::kStage);
  // Q fragments and the first tile have landed (the second may be in flight)
  if (AHEAD > 1 && nt > 1)
    wait_vm(std::integral_constant<int, C::kTileInst>{});
  else
    __builtin_amdgcn_s_waitcnt(0);

  // One tile.  The stage being filled and the one being read come in as
  // restrict-qualified parameters: the transpose reads of the current stage
  // then carry alias information that sets them apart from the loads issued
  // just before, so they need not wait for those loads (without it the
  // compiler waits for every outstanding direct-to-LDS load before a
  // transpose read, and the load latency of the tiles ahead lands in every
  // iteration).  The wait at the end of the tile keeps the order: the next
  // tile has landed before it is read.
  auto tile = [&](int t, uint16_t* __restrict__ nxt, const uint16_t* __restrict__ st) {
    const int j0 = (t_begin + t) * BN;
    // tile t + AHEAD streams into the stage that tile t - 1 used (this
    // wave's own: its reads finished when that tile's MFMAs took them)
    if (t + AHEAD < nt) issue_tile(j0 + AHEAD * BN, nxt);

    // S^T = K Q^T over two accumulators (even and odd k-steps), which halves
    // the chain of dependent MFMAs a single wave waits through
    auto compute_s = [&]() {
      f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NKS; ks += 2) {
        s0 = mfma_32x32x16<BF16>(*reinterpret_cast<const u32x4_t*>(st + k_rd + 16 * ks), qf[ks], s0);
        s1 = mfma_32x32x16<BF16>(*reinterpret_cast<const u32x4_t*>(st + k_rd + 16 * ks + 16),
                                 qf[ks + 1], s1);
      }
      f32x16_t sv = s0 + s1;
      if (prescale) sv *= c_log2;
      return sv;
    };
    // tile maximum (in-lane, then across the two lane halves); m is raised
    // when it is exceeded by more than `threshold`, and O and l follow
    auto raise_max = [&](const f32x16_t& sv, float threshold) {
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = max3(tmax, sv[r], sv[r + 1]);
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
    auto exponentiate = [&](f32x16_t& sv) {
      const float mb = m != -INFINITY ? m : 0.f;
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        sv[r] = exp2_fast(__builtin_fmaf(sv[r], ce, -mb));
        sv[r + 1] = exp2_fast(__builtin_fmaf(sv[r + 1], ce, -mb));
        ps0 += sv[r];
        ps1 += sv[r + 1];
      }
      return ps0 + ps1;
    };
    f32x16_t s = compute_s();
    const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > q0 + diag);
    float psum;
    if (t > 0 && !need_mask) {
      // Every row sees the whole tile and, having seen this wave's first
      // tile whole as well, has a finite m: exponentials against the current
      // m without a tile maximum.  A partial row sum above kSumLimit (a score
      // far above m, rare) takes the maximum path, with S recomputed from
      // the K tile still in LDS; one m enters l and O either way.
      psum = exponentiate(s);
      if (__builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) != 0) {
        s = compute_s();
        raise_max(s, 0.0f);
        psum = exponentiate(s);
      }
    } else {
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool vis = j < Nk && (!CAUSAL || j <= my_q + diag);
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
      raise_max(s, kRescale);
      psum = exponentiate(s);
    }
    lsum += psum;
    // O^T += V^T P^T; P as hi + lo halves where the tile crosses the diagonal
    auto pv = [&](auto with_lo) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        f32x8_t pvv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pvv[e] = s[8 * kk + e];
        const u32x4_t phi = pack8<BF16>(pvv);
        u32x4_t plo;
        if constexpr (decltype(with_lo)::value) plo = pack8<BF16>(pvv - unpack8<BF16>(phi));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2_t x0 = lds_read_tr4(st + v_rd + 16 * kk * VS + 32 * db);
          const u32x2_t x1 = lds_read_tr4(st + v_rd + (16 * kk + 8) * VS + 32 * db);
          const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
          oacc[db] = mfma_32x32x16<BF16>(a, phi, oacc[db]);
          if constexpr (decltype(with_lo)::value) oacc[db] = mfma_32x32x16<BF16>(a, plo, oacc[db]);
        }
      }
    };
    // (rows of a block whose first row sees fewer than 128 keys take the lo
    // half on every tile: there one P entry can carry most of a row's weight)
    if (CAUSAL && (need_mask || q0 + diag + 1 < 128))
      pv(std::true_type{});
    else
      pv(std::false_type{});
    // tile t + 1 has landed (vector memory operations retire in order; the
    // loads of tile t + 2, when issued, may stay in flight)
    if (AHEAD > 1 && t + 2 < nt)
      wait_vm(std::integral_constant<int, C::kTileInst>{});
    else
      __builtin_amdgcn_s_waitcnt(0);
  };
  for (int t = 0, cur = 0; t < nt; ++t) {
    const int nx = cur + AHEAD >= C::kStages ? cur + AHEAD - C::kStages : cur + AHEAD;
    tile(t, wst + nx * C::kStage, wst + cur * C::kStage);
    cur = cur + 1 == C::kStages ? 0 : cur + 1;
  }

  // ---- Merge the four waves' partial results through LDS.
  __syncthreads();  // every wave is done with its stages
  float* const mo = reinterpret_cast<float*>(smem);                // [wave][db][r][lane]
  float* const mm = mo + C::kWaves * BM * D;                       // [wave][lane] m
  float* const ml = mm + C::kWaves * 64;                           // [wave][lane] l (whole row)
  const float lrow = lsum + __shfl_xor(lsum, 32);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mo[((wave * NDB + db) * 16 + r) * 64 + lane] = oacc[db][r];
  }
  mm[wave * 64 + lane] = m;
  ml[wave * 64 + lane] = lrow;
  __syncthreads();

  // wave w merges O^T block db = w (d = 64 has two blocks: waves 0 and 1)
  float wts[C::kWaves];
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) Mx = __builtin_fmaxf(Mx, mm[w * 64 + lane]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < C::kWaves; ++w) {
    const float mw = mm[w * 64 + lane];
    wts[w] = mw != -INFINITY ? exp2_fast(mw - Mx) : 0.f;
    L += ml[w * 64 + lane] * wts[w];
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (wave < NDB) {
    const int db = wave;
    const rsrc_t orr = make_rsrc(O + qo_off, span_bytes(q0, BM, Nq, q_rs, D));
    const int ovoff = (int)(l32 * q_rs * 2) + 8 * hh;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4_t o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < C::kWaves; ++w) acc += mo[((w * NDB + db) * 16 + 4 * g + e) * 64 + lane] * wts[w];
        o4[e] = acc * inv;
      }
      buf_store8(pack4<BF16>(o4), orr, ovoff + 2 * (32 * db + 8 * g));
    }
  }
  if (wave == 0) {
    const int nrows = max(0, min(BM, Nq - q0));
    const rsrc_t lr = make_rsrc(LSE + ((int64_t)b * Hq + hq) * Nq + q0, nrows * 4);
    if (hh == 0) buf_store4(L > 0.f ? (Mx + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY, lr, 4 * l32);
  }
}

}  // namespace eta
