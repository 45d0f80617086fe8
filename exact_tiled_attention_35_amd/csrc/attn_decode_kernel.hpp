// KV-cache decode forward for gfx950 (MI355X, CDNA4).
//
// The inference path of the hysenlabs.com page "FlashAttention: exakte
// Attention-Kernel fuer CUDA und ROCm" (section "Die Schnittstellen von
// flash_attn_func bis KV-Cache"): a few new query rows attend to a long
// key/value cache; the new keys and values are written into the cache in
// place first, and there is no backward pass.  Per batch b the cache holds
// cache_seqlens[b] valid rows before the append and cache_seqlens[b] + Nnew
// after it; the query rows attend to all of those (causal: bottom-right
// aligned, as everywhere in this library).
//
// Kernels:
//  * kv_append_kernel: copies k_new / v_new rows into the cache at row
//    cache_seqlens[b] + t (16 bytes per thread); used only when there are no
//    query rows (Nq = 0).  Otherwise attn_decode_kernel appends them itself:
//    the tiles that hold new rows take them from k_new / v_new, and the
//    workgroups of the first row block write them to the cache.
//  * attn_decode_kernel: one workgroup per (b, KV head, block of 128 packed
//    query rows, key split).  The query heads of a GQA group are packed into
//    the rows of one MFMA tile (packed row r = (head g*G + r / Nq, query
//    r % Nq)), so each KV head's cache is streamed once per split for the
//    whole group.  The keys of (b, KV head) are cut into `splits` ranges of
//    whole tiles, one per workgroup, so that short query blocks still fill
//    the GPU; K/V tiles stream through two LDS stages (the loop is bound by
//    HBM, not by the matrix cores).  The
//    products, the online softmax and the masking are the forward kernel's
//    (S^T = K Q^T and O^T = V^T P^T on 32x32x16 MFMAs, one query row per
//    lane, exp2 with the running maximum).  With one split the result goes
//    straight to out/lse; otherwise each workgroup writes its normalised
//    fp32 partial O and its logsumexp to the workspace.
//  * attn_decode_merge_kernel: per query row, lse = log sum_s exp(lse_s) and
//    O = sum_s exp(lse_s - lse) O_s -- the same merge that combines key
//    ranges across devices.
#pragma once

#include <type_traits>

#include "gfx950_ops.hpp"

namespace eta {

template <int D>
struct DecCfg {
  static constexpr int kWaves = 4, kThreads = 256, BM = 128;
  static constexpr int BN = 32;       // keys per tile
  static constexpr int kStages = 2;   // the next tile streams in while this one is computed
  static constexpr int kChunks = D / 8;
  static constexpr int KCP = kChunks + 1, VCP = kChunks + 4;
  static constexpr int KS = 8 * KCP, VS = 8 * VCP;
  static constexpr int kKInst = (BN * KCP + 63) / 64, kVInst = (BN * VCP + 63) / 64;
  static constexpr int kKElems = kKInst * 512, kVElems = kVInst * 512;
  static constexpr int kStage = kKElems + kVElems;
  static constexpr int kLdsElems = kStages * kStage;
  static constexpr int kKInstPerWave = (kKInst + 3) / 4, kVInstPerWave = (kVInst + 3) / 4;
  static constexpr int kMinWavesPerEU = (D >= 256) ? 1 : 2;
  static_assert((KS / 2) % 8 == 4 && (VS / 2) % 32 == 16, "bank-conflict-free strides");
};

// Appends Nnew rows per (b, KV head) to the caches: row cache_seqlens[b] + t.
// Rows that would land at or past Ncap are dropped (the range of the
// destination descriptor ends there).
template <int D>
__global__ void __launch_bounds__(256)
kv_append_kernel(const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vn,
                 uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc,
                 const int* __restrict__ seqlens, int B, int Nnew, int Hkv, int Ncap) {
  constexpr int kChunks = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)B * Nnew * Hkv * kChunks;
  if (idx >= total) return;
  const int c = (int)(idx % kChunks);
  const int64_t row = idx / kChunks;  // (b, t, h) of the new rows
  const int h = (int)(row % Hkv);
  const int t = (int)((row / Hkv) % Nnew);
  const int b = (int)(row / ((int64_t)Hkv * Nnew));
  const int pos = seqlens[b] + t;
  const int64_t cache_b = (int64_t)b * Ncap * Hkv * D;
  const int cache_bytes = (int)((int64_t)Ncap * Hkv * D * 2);
  const int dst = pos >= 0 && pos < Ncap ? (int)((((int64_t)pos * Hkv + h) * D + 8 * c) * 2) : cache_bytes;
  const int src = (int)((row * D + 8 * c) * 2);
  const rsrc_t kn = make_rsrc(Kn, (int)(total * 16)), vn = make_rsrc(Vn, (int)(total * 16));
  const rsrc_t kc = make_rsrc(Kc + cache_b, cache_bytes), vc = make_rsrc(Vc + cache_b, cache_bytes);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(kn, src, 0, 0), kc, dst, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(vn, src, 0, 0), vc, dst, 0, 0);
}

template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(DecCfg<D>::kThreads, DecCfg<D>::kMinWavesPerEU)
attn_decode_kernel(const uint16_t* __restrict__ Q, uint16_t* __restrict__ K,
                   uint16_t* __restrict__ V, const int* __restrict__ seqlens,
                   const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vn,
                   uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart,
                   float* __restrict__ Lpart, int B, int Hq, int Hkv, int Nq, int Ncap, int Nnew,
                   int nrb, int splits, float c_log2, int prescale) {
  using C = DecCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NKS = D / 16, NKB = BN / 32, NDB = D / 32, NKK = BN / 16;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::kLdsElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // blockIdx -> (b, KV head, row block, split).
  int lid = blockIdx.x;
  const int s = lid % splits;
  lid /= splits;
  const int rb = lid % nrb;
  lid /= nrb;
  const int hkv = lid % Hkv;
  const int b = lid / Hkv;
  const int G = Hq / Hkv;
  const int rows = G * Nq;

  // This lane's packed row -> (query head, query row).
  const int rw0 = rb * BM + wave * 32;
  const int r = rw0 + l32;
  const bool row_ok = r < rows;
  const int h = hkv * G + (row_ok ? r / Nq : 0);
  const int i = row_ok ? r % Nq : 0;
  const bool wave_live = rw0 < rows;

  // Keys of batch b and of this split (whole tiles).  Rows [sl_b, nk) are
  // the new ones (row sl_b + t of the cache is new row t, clipped to Ncap).
  const int sl_b = seqlens[b];
  const int nk = min(Ncap, max(0, sl_b + Nnew));
  const int diag = nk - Nq;
  const int tiles = (nk + BN - 1) / BN;
  const int tps = (tiles + splits - 1) / splits;
  const int t0 = min(tiles, s * tps), t1 = min(tiles, t0 + tps);
  // (Causal never shortens the range: query row Nq - 1 sees every key.)
  const int kv_end = min(nk, t1 * BN);
  const int nt = kv_end > t0 * BN ? (kv_end - t0 * BN + BN - 1) / BN : 0;

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  uint16_t* const Kh = K + ((int64_t)b * Ncap * Hkv + hkv) * D;
  uint16_t* const Vh = V + ((int64_t)b * Ncap * Hkv + hkv) * D;

  // Q^T fragments of this lane's row; rows past the packed rows read 0.
  const int qbytes = (int)((int64_t)Nq * q_rs * 2);
  const rsrc_t qr = make_rsrc(Q + (int64_t)b * Nq * q_rs, qbytes);
  const int qoff = row_ok ? (int)(((int64_t)i * q_rs + (int64_t)h * D) * 2) + 16 * hh : qbytes;
  u32x4_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qr, qoff + (row_ok ? 32 * ks : 0));

  int koff[C::kKInstPerWave], voff[C::kVInstPerWave];
#pragma unroll
  for (int k = 0; k < C::kKInstPerWave; ++k) {
    const int sl = 64 * (wave + 4 * k) + lane;
    const int row = min(sl / C::KCP, BN - 1), c = min(sl % C::KCP, C::kChunks - 1);
    koff[k] = (int)(row * kv_rs * 2) + 16 * c;
  }
#pragma unroll
  for (int k = 0; k < C::kVInstPerWave; ++k) {
    const int sl = 64 * (wave + 4 * k) + lane;
    const int row = min(sl / C::VCP, BN - 1), c = min(sl % C::VCP, C::kChunks - 1);
    voff[k] = (int)(row * kv_rs * 2) + 16 * c;
  }
  auto issue_tile = [&](int t, uint16_t* st) {
    const int j0 = (t0 + t) * BN;
    const int bytes = span_bytes(j0, BN, nk, kv_rs, D);
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, bytes);
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, bytes);
#pragma unroll
    for (int k = 0; k < C::kKInstPerWave; ++k) {
      const int j = wave + 4 * k;
      if (j < C::kKInst) buf_load_lds16(kr, st + 512 * j, koff[k]);
    }
#pragma unroll
    for (int k = 0; k < C::kVInstPerWave; ++k) {
      const int j = wave + 4 * k;
      if (j < C::kVInst) buf_load_lds16(vr, st + C::kKElems + 512 * j, voff[k]);
    }
  };

  const int g16 = lane >> 4, i16 = lane & 15;
  const int k_rd = l32 * KS + 8 * hh;
  const int v_rd = C::kKElems + (4 * hh + (i16 >> 2)) * VS + 16 * (g16 & 1) + 4 * (i16 & 3);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;
  const float ce = prescale ? 1.0f : c_log2;

  // Two LDS stages.  The V reads of a tile wait for every load this wave
  // has in flight (the compiler cannot tell the stages apart), so deeper
  // rings keep no more loads in flight; a four-stage ring with waits on
  // the older tiles only was measured slower on this HBM stream.
  if (nt > 0) issue_tile(0, smem);

  for (int t = 0; t < nt; ++t) {
    // Tile t has landed: every wave waits for its own loads, then the
    // barrier publishes them and ends all reads of the stage the next tile
    // reuses (read in iteration t - 1).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < nt) issue_tile(t + 1, smem + ((t + 1) & 1) * C::kStage);
    const uint16_t* st = smem + (t & 1) * C::kStage;
    const int j0 = (t0 + t) * BN;
    // The new rows of this tile come from k_new / v_new: they replace what
    // the tile load brought from those cache rows (which another workgroup
    // may be writing just now), and the workgroups of the first row block
    // write them to the cache (each cache row belongs to one split).
    // Workgroup-uniform; at most a few tiles per call.
    const int new_lo = max(sl_b, j0), new_hi = min(nk, j0 + BN);
    if (new_lo < new_hi) {
      uint16_t* const sw = smem + (t & 1) * C::kStage;
      const int items = (new_hi - new_lo) * C::kChunks;
      for (int it = tid; it < items; it += C::kThreads) {
        const int pos = new_lo + it / C::kChunks, c = it % C::kChunks;
        const int64_t src = (((int64_t)b * Nnew + (pos - sl_b)) * Hkv + hkv) * D + 8 * c;
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(Kn + src);
        const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(Vn + src);
        *reinterpret_cast<u32x4_t*>(sw + (pos - j0) * KS + 8 * c) = kv;
        *reinterpret_cast<u32x4_t*>(sw + C::kKElems + (pos - j0) * VS + 8 * c) = vv;
        if (rb == 0) {
          *reinterpret_cast<u32x4_t*>(Kh + (int64_t)pos * kv_rs + 8 * c) = kv;
          *reinterpret_cast<u32x4_t*>(Vh + (int64_t)pos * kv_rs + 8 * c) = vv;
        }
      }
      __syncthreads();
    }

    if (wave_live) {
      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc[kb] = mfma_32x32x16<BF16>(
              *reinterpret_cast<const u32x4_t*>(st + k_rd + kb * 32 * KS + 16 * ks), qf[ks], sacc[kb]);
      }
      if (prescale) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sacc[kb] *= c_log2;
      }
      // Mask keys past the end and (causal) above the diagonal.
      const bool need_mask = (j0 + BN > kv_end) || CAUSAL;
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (need_mask) {
            const int j = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
            const bool vis = j < kv_end && (!CAUSAL || j <= i + diag);
            sacc[kb][e] = vis ? sacc[kb][e] : -INFINITY;
          }
          tmax = __builtin_fmaxf(tmax, sacc[kb][e]);
        }
      }
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
      const float tm = tmax * ce;
      if (tm > m) {
        const float alpha = exp2_fast(m - tm);
        m = tm;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }
      const float mb = m == -INFINITY ? 0.f : m;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(__builtin_fmaf(sacc[kb][e], ce, -mb));
          sacc[kb][e] = p;
          ps += p;
        }
      }
      lsum += ps;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        f32x8_t pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sacc[kk >> 1][8 * (kk & 1) + e];
        const u32x4_t phi = pack8<BF16>(pv), plo = pack8<BF16>(pv - unpack8<BF16>(phi));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2_t x0 = lds_read_tr4(st + v_rd + 16 * kk * VS + 32 * db);
          const u32x2_t x1 = lds_read_tr4(st + v_rd + (16 * kk + 8) * VS + 32 * db);
          const u32x4_t a = {x0[0], x0[1], x1[0], x1[1]};
          oacc[db] = mfma_32x32x16<BF16>(a, phi, oacc[db]);
          oacc[db] = mfma_32x32x16<BF16>(a, plo, oacc[db]);
        }
      }
    }
  }

  // Epilogue: this split's normalised output and natural-log logsumexp.
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  const int64_t row_id = ((int64_t)b * Hq + h) * Nq + i;  // [B, Hq, Nq] order
  if (splits == 1) {
    const int obytes = (int)((int64_t)Nq * q_rs * 2);
    const rsrc_t orr = make_rsrc(O + (int64_t)b * Nq * q_rs, obytes);
    const int ooff = (int)(((int64_t)i * q_rs + (int64_t)h * D) * 2) + 8 * hh;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * inv;
        buf_store8(pack4<BF16>(o4), orr, ooff + 2 * (32 * db + 8 * g));
      }
    }
    if (hh == 0) LSE[row_id] = lse;
  } else {
    const int64_t prow = (int64_t)s * B * Hq * Nq + row_id;
    float* op = Opart + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4_t*>(op + 32 * db + 8 * g + 4 * hh) = o4;
      }
    }
    if (hh == 0) Lpart[prow] = lse;
  }
}

// One wave per query row: lse = log sum_s exp(lse_s), O = sum_s w_s O_s with
// w_s = exp(lse_s - lse); rows no split saw get O = 0 and lse = -inf.  Lane
// l holds the logsumexp of splits l and 64 + l, so the maximum and the
// sum of the weights take two loads and a few lane exchanges.  The partial
// outputs are read 16 bytes per lane: a wave covers 64 / (D / 4) splits per
// load, each lane recomputes its split's weight, the loads of all splits are
// independent, and the lane groups that summed different splits are added at
// the end.
template <int D, bool BF16>
__global__ void __launch_bounds__(256)
attn_decode_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                         uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Nq,
                         int splits) {
  constexpr int CPR = D / 4;        // 16-byte chunks per row
  constexpr int SPL = 64 / CPR;     // splits per load instruction
  const int64_t nrow = (int64_t)B * Hq * Nq;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrow) return;  // the whole wave
  // splits <= 128: lane l covers splits l and 64 + l
  const float ls0 = lane < splits ? Lpart[(int64_t)lane * nrow + row] : -INFINITY;
  const float ls1 = 64 + lane < splits ? Lpart[(int64_t)(64 + lane) * nrow + row] : -INFINITY;
  float mx = __builtin_fmaxf(ls0, ls1);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, x));
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  const int sub = lane / CPR, c = lane % CPR;
  if (mx != -INFINITY) {
    const float w0 = ls0 == -INFINITY ? 0.f : exp2_fast((ls0 - mx) * 1.44269504088896340736f);
    const float w1 = ls1 == -INFINITY ? 0.f : exp2_fast((ls1 - mx) * 1.44269504088896340736f);
    den = w0 + w1;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) den += __shfl_xor(den, x);
    const f32x4_t* op = reinterpret_cast<const f32x4_t*>(Opart + row * D) + c;
    const int64_t split_stride = nrow * CPR;  // in 16-byte chunks
    // CH splits per lane at a time: all their loads first, then the sums.
    constexpr int CH = 16;
    for (int s0 = 0; s0 < splits; s0 += SPL * CH) {
      float lsv[CH];
      f32x4_t vv[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        // this lane's split; past the last one, reread it with weight 0
        const int sp = min(s0 + SPL * u + sub, splits - 1);
        lsv[u] = Lpart[(int64_t)sp * nrow + row];
        vv[u] = op[sp * split_stride];
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const bool live = s0 + SPL * u + sub < splits && lsv[u] != -INFINITY;
        const float wgt = live ? exp2_fast((lsv[u] - mx) * 1.44269504088896340736f) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wgt, vv[u][e], acc[e]);
      }
    }
#pragma unroll
    for (int x = CPR; x < 64; x <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], x);
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  // row = (b * Hq + h) * Nq + i -> out[b, i, h, :]
  const int i = (int)(row % Nq);
  const int64_t bh = row / Nq;
  const int h = (int)(bh % Hq);
  const int64_t b = bh / Hq;
  if (sub == 0) {
    f32x4_t o4;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = acc[e] * inv;
    *reinterpret_cast<u32x2_t*>(O + ((b * Nq + i) * Hq + h) * D + 4 * c) = pack4<BF16>(o4);
  }
  if (lane == 0) LSE[row] = den > 0.f ? mx + __builtin_amdgcn_logf(den) * kLn2 : -INFINITY;
}

}  // namespace eta
