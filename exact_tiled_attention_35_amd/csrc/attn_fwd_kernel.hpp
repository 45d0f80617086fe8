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

// max(max(a, b), c): one v_max3_f32.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Raw buffer resources.  Every global access goes through a descriptor whose
// range covers exactly the valid rows of the current tile: the hardware
// returns 0 for loads past the range and drops stores past it, so ragged
// tails need no branches, and per-thread byte offsets stay loop-invariant
// (only the scalar base address moves from tile to tile).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__device__ __forceinline__ void buf_store8(u32x2_t v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}

__device__ __forceinline__ void buf_store4(float v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, 0, 0);
}

// Bytes from row r0 to the end of the last valid row of a [rows, D] window
// of a tensor with row stride rs (elements), given N valid rows in total.
__device__ __forceinline__ int span_bytes(int r0, int rows, int N, int64_t rs, int D) {
  const int valid = min(rows, N - r0);
  return valid > 0 ? (int)(((int64_t)(valid - 1) * rs + D) * 2) : 0;
}

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const WorkItem w = map_workgroup<CAUSAL>(blockIdx.x, total, nqb, Hq);
  const int hkv = w.hq / (Hq / Hkv);
  const int q0 = w.qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const int diag = Nk - Nq;  // causal: key j visible to row i iff j <= i + diag

  const int64_t q_rs = (int64_t)Hq * D, kv_rs = (int64_t)Hkv * D;
  // Row qw0 of (b, hq) in q / out; row 0 of (b, hkv) in k / v.
  const int64_t qo_off = ((int64_t)w.b * Nq + qw0) * q_rs + (int64_t)w.hq * D;
  const uint16_t* Kh = K + ((int64_t)w.b * Nk * Hkv + hkv) * D;
  const uint16_t* Vh = V + ((int64_t)w.b * Nk * Hkv + hkv) * D;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop.
  u32x4_t qf[NKS];
  {
    const rsrc_t qr = make_rsrc(Q + qo_off, span_bytes(qw0, 32, Nq, q_rs, D));
    const int voff = (int)(l32 * q_rs * 2) + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qr, voff + 32 * ks);
  }

  // ---- Key range of the workgroup and of this wave.
  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, min(q0 + BM, Nq) + diag);
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int rows_end = min(qw0 + 32, Nq);
  int w_end = rows_end > qw0 ? Nk : 0;
  if (CAUSAL && rows_end > qw0) w_end = min(Nk, rows_end + diag);

  // ---- Tile staging: global -> registers -> LDS, with loop-invariant offsets.
  int koff[C::kKChunksPerThread], kls[C::kKChunksPerThread];
#pragma unroll
  for (int i = 0; i < C::kKChunksPerThread; ++i) {
    const int c = tid + C::kThreads * i;
    const int row = c / KCPR, cc = c % KCPR;
    koff[i] = (int)(row * kv_rs * 2) + 16 * cc;
    kls[i] = row * KS + 8 * cc;
  }
  int voff[C::kVBlocksPerThread][4], vls[C::kVBlocksPerThread];
#pragma unroll
  for (int i = 0; i < C::kVBlocksPerThread; ++i) {
    // Consecutive lanes take consecutive 4-key groups of one 8-column chunk:
    // the lanes of one LDS write pass then fill one V^T row without bank
    // conflicts, and each global load still reads whole 64-byte runs.
    const int blk = tid + C::kThreads * i;
    const int kg = blk % (BN / 4);
    const int cc = blk / (BN / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) voff[i][j] = (int)((4 * kg + j) * kv_rs * 2) + 16 * cc;
    vls[i] = C::kKElems + (8 * cc) * VS + vt_pos(4 * kg);
  }
  // V blocks exist for whole waves only (kVBlocks is a multiple of 64).
  auto has_vblock = [&](int i) {
    return (C::kVBlocks % C::kThreads == 0) || (wave * 64 + C::kThreads * i < C::kVBlocks);
  };

  u32x4_t kreg[C::kKChunksPerThread];
  u32x4_t vreg[C::kVBlocksPerThread][4];

  auto load_tile = [&](int j0) {
    const int bytes = span_bytes(j0, BN, Nk, kv_rs, D);
    const rsrc_t kr = make_rsrc(Kh + (int64_t)j0 * kv_rs, bytes);
    const rsrc_t vr = make_rsrc(Vh + (int64_t)j0 * kv_rs, bytes);
#pragma unroll
    for (int i = 0; i < C::kKChunksPerThread; ++i) kreg[i] = buf_load16(kr, koff[i]);
#pragma unroll
    for (int i = 0; i < C::kVBlocksPerThread; ++i) {
      if (has_vblock(i)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[i][j] = buf_load16(vr, voff[i][j]);
      }
    }
  };

  auto store_tile = [&](uint16_t* st) {
#pragma unroll
    for (int i = 0; i < C::kKChunksPerThread; ++i)
      *reinterpret_cast<u32x4_t*>(st + kls[i]) = kreg[i];
#pragma unroll
    for (int i = 0; i < C::kVBlocksPerThread; ++i) {
      if (has_vblock(i)) {
        uint16_t* dst = st + vls[i];
#pragma unroll
        for (int p = 0; p < 4; ++p) {  // element pair (2p, 2p+1) of the 8 columns
          const uint32_t r0 = vreg[i][0][p], r1 = vreg[i][1][p];
          const uint32_t r2 = vreg[i][2][p], r3 = vreg[i][3][p];
          u32x2_t even, odd;
          even[0] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);
          even[1] = __builtin_amdgcn_perm(r3, r2, 0x05040100u);
          odd[0] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
          odd[1] = __builtin_amdgcn_perm(r3, r2, 0x07060302u);
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

  // Tile 0 is staged even when no tile is needed (nt == 0): the access is in
  // range (Nk >= 1), and it leaves no load outstanding when the loop starts.
  load_tile(0);
  store_tile(smem);
  __builtin_amdgcn_s_waitcnt(0);  // Q fragments and tile 0 have landed
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
        for (int r = 0; r < 16; r += 2) tmax = max3(tmax, s[kb][r], s[kb][r + 1]);
      }
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
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

  // ---- Epilogue: normalise, round, store O and the logsumexp.  Stores of
  // rows >= Nq fall outside the descriptors' ranges and are dropped.
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const rsrc_t orr = make_rsrc(O + qo_off, span_bytes(qw0, 32, Nq, q_rs, D));
  const int ovoff = (int)(l32 * q_rs * 2) + 8 * hh;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4_t o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * inv;
      buf_store8(pack4<BF16>(o4), orr, ovoff + 2 * (32 * db + 8 * g));
    }
  }
  const int nrows = max(0, min(32, Nq - qw0));
  const rsrc_t lr = make_rsrc(LSE + ((int64_t)w.b * Hq + w.hq) * Nq + qw0, nrows * 4);
  buf_store4(lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY, lr, 4 * l32);
}

}  // namespace eta
