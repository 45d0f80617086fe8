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
//        S^T = K . Q^T   (A = K tile from LDS, B = Q^T kept in VGPRs)
//        O^T = V^T . P^T (A = V^T tile from LDS, B = P^T straight from the
//                         S^T accumulators)
//    With the 32x32 accumulator layout (lane l, register r holds row
//    8*(r/4) + 4*(l/32) + r%4, column l%32), column = query, so every lane owns
//    ONE query row: the running max / sum / rescale factor are per-lane
//    scalars and a row reduction is an in-lane reduction plus one exchange
//    between lanes l and l+32.
//  * K tiles are staged row-major in LDS, V tiles transposed (d-major) with
//    the keys of each 16-key group stored in the order that makes one lane's
//    8 B-operand keys one contiguous 16-byte LDS read.  Rows are padded by
//    16 bytes so that 16 consecutive lanes reading 16 different rows hit
//    distinct banks.  K/V tiles are double-buffered: the global loads of tile
//    t+1 are in flight while tile t is computed, one barrier per tile.
//  * Online softmax in the log2 domain: t = s * scale * log2(e), p = 2^(t - m).
//    The running maximum m is only raised when a tile's maximum exceeds it
//    by more than RESCALE_THRESHOLD (p then stays <= 2^threshold).  Because
//    the same m is used for the sum l and for O, the result is still exact;
//    the rescale of O is skipped on almost every tile.
//  * Causal: tiles entirely above the diagonal are never loaded; tiles that
//    cross it (and ragged tails) are masked per element.  On those tiles P is
//    fed to the PV product as hi + lo halves (two MFMAs), which keeps the
//    early causal rows -- where one P entry carries most of the weight -- at
//    the accuracy of the output rounding.
//  * The row sum l is accumulated from the unrounded fp32 p.
//  * Epilogue: O /= l, rounded to nearest-even; lse = (m + log2 l) * ln 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eta {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p <= 256 between rescales

// Tile shape per head dimension.
template <int D>
struct TileCfg {
  static constexpr int kWaves = 4;
  static constexpr int BM = 32 * kWaves;                 // query rows per workgroup
  static constexpr int BN = (D >= 256) ? 32 : 64;        // keys per K/V tile
  static constexpr int KS = D + 8;                       // K row stride in LDS (elements)
  static constexpr int VS = BN + 8;                      // V^T row stride in LDS (elements)
  static constexpr int kKElems = BN * KS;
  static constexpr int kVElems = D * VS;
  static constexpr int kStage = kKElems + kVElems;       // one LDS buffer (elements)
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKChunks = BN * D / 8;            // 16-byte chunks per K tile
  static constexpr int kKChunksPerThread = kKChunks / kThreads;
  static constexpr int kVBlocks = BN * D / 32;           // 4 keys x 8 columns per block
  static constexpr int kVBlocksPerThread = (kVBlocks + kThreads - 1) / kThreads;
  static constexpr int kMinWavesPerEU = (D >= 256) ? 1 : 2;
  static_assert(kKChunks % kThreads == 0, "K tile must split evenly over the workgroup");
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile sizes must be multiples of 32");
};

template <bool BF16>
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Round 8 floats to the element type (nearest-even) and pack them.
template <bool BF16>
__device__ __forceinline__ u32x4_t pack8(f32x8_t x) {
  if constexpr (BF16) {
    return __builtin_bit_cast(u32x4_t, __builtin_convertvector(x, bf16x8_t));
  } else {
    return __builtin_bit_cast(u32x4_t, __builtin_convertvector(x, f16x8_t));
  }
}

template <bool BF16>
__device__ __forceinline__ u32x2_t pack4(f32x4_t x) {
  if constexpr (BF16) {
    return __builtin_bit_cast(u32x2_t, __builtin_convertvector(x, bf16x4_t));
  } else {
    return __builtin_bit_cast(u32x2_t, __builtin_convertvector(x, f16x4_t));
  }
}

// Widen 8 packed elements back to fp32 (exact).
template <bool BF16>
__device__ __forceinline__ f32x8_t unpack8(u32x4_t x) {
  if constexpr (BF16) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8_t, x), f32x8_t);
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x8_t, x), f32x8_t);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of key k (within a tile) in a V^T row: bits 2 and 3 of k are
// swapped, so keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key group -- the keys
// lane half h feeds to one PV MFMA -- are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

// Work item of one workgroup.
struct WorkItem {
  int b, hq, qblk;
};

// blockIdx -> (b, head, query block).  Workgroups are handed to the 8 XCDs
// round-robin, so the logical order is regrouped to give each XCD a
// contiguous run of (b, head) pairs: all query blocks of a head (and the
// query heads of one GQA group, which are adjacent) then share one XCD's L2.
// Causal launches run the longest query blocks first.
template <bool CAUSAL>
__device__ __forceinline__ WorkItem map_workgroup(int wg, int total, int nqb, int Hq) {
  int lid = wg;
  if ((total & 7) == 0) lid = (wg & 7) * (total >> 3) + (wg >> 3);
  WorkItem w;
  w.qblk = lid % nqb;
  const int bh = lid / nqb;
  w.hq = bh % Hq;
  w.b = bh / Hq;
  if (CAUSAL) w.qblk = nqb - 1 - w.qblk;
  return w;
}

template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(TileCfg<D>::kThreads, TileCfg<D>::kMinWavesPerEU)
attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, int nqb,
                int total, float c_log2, int prescale) {
  using C = TileCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, VS = C::VS;
  constexpr int NKS = D / 16;  // k-steps of the S^T product
  constexpr int NKB = BN / 32; // 32-key blocks per tile
  constexpr int NDB = D / 32;  // 32-column blocks of O^T
  constexpr int NKK = BN / 16; // 16-key steps of the PV product
  constexpr int KCPR = D / 8;  // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::kStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const WorkItem w = map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const int diag = Nk - Nq;  // causal: key j visible to row i iff j <= i + diag

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  const uint16_t* Qb = Q + ((int64_t)w.b * Nq * Hq + w.hq) * D;
  const uint16_t* Kb = K + ((int64_t)w.b * Nk * Hkv + hkv) * D;
  const uint16_t* Vb = V + ((int64_t)w.b * Nk * Hkv + hkv) * D;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop.
  u32x4_t qf[NKS];
  {
    const bool in = my_q < Nq;
    const uint16_t* qrow = Qb + (int64_t)(in ? my_q : 0) * q_rs + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = in ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- Key range of the workgroup and of this wave.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);

  // ---- Tile staging: global -> registers -> LDS.
  u32x4_t kreg[C::kKChunksPerThread];
  u32x4_t vreg[C::kVBlocksPerThread][4];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < C::kKChunksPerThread; ++i) {
      const int c = tid + C::kThreads * i;
      const int row = c / KCPR, cc = c % KCPR;
      const int key = j0 + row;
      kreg[i] = key < Nk ? *reinterpret_cast<const u32x4_t*>(Kb + (int64_t)key * kv_rs + 8 * cc)
                         : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::kVBlocksPerThread; ++i) {
      const int blk = tid + C::kThreads * i;
      const int cc = (blk & 3) + 4 * ((blk >> 2) / (BN / 4));
      const int kg = (blk >> 2) % (BN / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = j0 + 4 * kg + j;
        vreg[i][j] = (blk < C::kVBlocks && key < Nk)
                         ? *reinterpret_cast<const u32x4_t*>(Vb + (int64_t)key * kv_rs + 8 * cc)
                         : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](uint16_t* Ks) {
    uint16_t* Vs = Ks + C::kKElems;
#pragma unroll
    for (int i = 0; i < C::kKChunksPerThread; ++i) {
      const int c = tid + C::kThreads * i;
      const int row = c / KCPR, cc = c % KCPR;
      *reinterpret_cast<u32x4_t*>(Ks + row * KS + 8 * cc) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::kVBlocksPerThread; ++i) {
      const int blk = tid + C::kThreads * i;
      if (blk < C::kVBlocks) {
        const int cc = (blk & 3) + 4 * ((blk >> 2) / (BN / 4));
        const int kg = (blk >> 2) % (BN / 4);
        uint16_t* dst = Vs + (8 * cc) * VS + vt_pos(4 * kg);
#pragma unroll
        for (int p = 0; p < 4; ++p) {  // element pair (2p, 2p+1) of the 8 columns
          const uint32_t r0 = vreg[i][0][p], r1 = vreg[i][1][p];
          const uint32_t r2 = vreg[i][2][p], r3 = vreg[i][3][p];
          u32x2_t even, odd;
          even[0] = (r0 & 0xffffu) | (r1 << 16);
          even[1] = (r2 & 0xffffu) | (r3 << 16);
          odd[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          odd[1] = (r2 >> 16) | (r3 & 0xffff0000u);
          *reinterpret_cast<u32x2_t*>(dst + (2 * p) * VS) = even;
          *reinterpret_cast<u32x2_t*>(dst + (2 * p + 1) * VS) = odd;
        }
      }
    }
  };

  // ---- Running state (per lane = per query row).
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m = -INFINITY;  // running max of t = s * c_log2 (log2 units)
  float lsum = 0.f;     // this lane half's share of the running sum
  const float ce = prescale ? 1.0f : c_log2;

  if (nt > 0) {
    load_tile(0);
    store_tile(smem);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int j0 = t * BN;
    if (t + 1 < nt) load_tile(j0 + BN);
    const uint16_t* Ks = smem + (t & 1) * C::kStage;
    const uint16_t* Vs = Ks + C::kKElems;

    if (j0 < w_end) {  // wave-uniform: skip tiles above this wave's diagonal
      // S^T = K Q^T for BN keys x 32 queries.
      f32x16_t s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(Ks + (kb * 32 + l32) * KS + 16 * ks + 8 * hh);
          s[kb] = mfma_32x32x16<BF16>(a, qf[ks], s[kb]);
        }
      }
      if (prescale) {  // scale <= 0: take the max of s*c directly
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] *= c_log2;
      }

      // Mask keys past the end and (causal) above the diagonal.
      const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > qw0 + diag);
      if (need_mask) {
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

      // Tile row maximum: in-lane, then across the two lane halves.
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) tmax = fmaxf(tmax, fmaxf(s[kb][r], s[kb][r + 1]));
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float tm = tmax * ce;
      if (tm > m + kRescaleThreshold) {  // raise m; rescale what was accumulated
        const float alpha = exp2_fast(m - tm);
        m = tm;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }
      const float mb = (m == -INFINITY) ? 0.f : m;

      // p = 2^(s*c - m); partial row sums from the unrounded p.
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
      lsum += ps0 + ps1;

      // O^T += V^T P^T.  One 16-key step uses registers 8*(kk%2)..+7 of
      // S^T block kk/2: keys {4hh..4hh+3, 8+4hh..8+4hh+3} of the 16-group.
      const bool split = CAUSAL && need_mask;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int kb = kk >> 1, r0 = 8 * (kk & 1);
        f32x8_t pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[kb][r0 + e];
        const u32x4_t phi = pack8<BF16>(pv);
        u32x4_t plo = u32x4_t{0, 0, 0, 0};
        if (split) plo = pack8<BF16>(pv - unpack8<BF16>(phi));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(Vs + (db * 32 + l32) * VS + 16 * kk + 8 * hh);
          oacc[db] = mfma_32x32x16<BF16>(a, phi, oacc[db]);
          if (split) oacc[db] = mfma_32x32x16<BF16>(a, plo, oacc[db]);
        }
      }
    }

    if (t + 1 < nt) store_tile(smem + ((t + 1) & 1) * C::kStage);
    __syncthreads();
  }

  // ---- Epilogue: normalise, round, store O and the logsumexp.
  const float lt = lsum + __shfl_xor(lsum, 32);
  if (my_q < Nq) {
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    uint16_t* orow = O + (((int64_t)w.b * Nq + my_q) * Hq + w.hq) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * inv;
        *reinterpret_cast<u32x2_t*>(orow + 32 * db + 8 * g) = pack4<BF16>(o4);
      }
    }
    if (hh == 0) {
      LSE[((int64_t)w.b * Hq + w.hq) * Nq + my_q] =
          lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace eta
