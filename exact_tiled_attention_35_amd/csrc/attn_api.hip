// C ABI of the exact tiled attention forward, the status strings and the
// version (declared in include/attn.h); the backward is in attn_bwd_api.hip.
//
// Host side only: argument validation (before any HIP call), a cached
// per-device gfx950 check, choice of the kernel instance, grid size, and the
// asynchronous launch on the caller's stream.  No device memory is allocated.

#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd_kernel.hpp"
#include "attn_fwd_k16_kernel.hpp"
#include "attn_fwd_splitk_kernel.hpp"
#include "attn_host.hpp"

namespace {

using eta_host::aligned16;
using eta_host::check_device;
using eta_host::finite_bits;
using eta_host::overlaps;

constexpr const char* kVersion = "0.3.0 gfx950 exact-tiled-attention fwd+bwd";
constexpr int kSmallGrid = 128;  // 128-row workgroups below which attn_fwd splits the keys

template <int D, bool BF16, bool CAUSAL, bool MODS, bool VARLEN = false, bool SPARSE = false>
int launch(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
           int Hkv, int Nq, int Nk, float scale, const eta::ScoreMods& mods, hipStream_t stream,
           const eta::VarlenArgs& va = eta::VarlenArgs{nullptr, nullptr, 0, 0, 0},
           const eta::BlockMaskArgs& bm = eta::BlockMaskArgs{nullptr, 0, 0}) {
  using C = eta::TileCfg<D>;
  const int nqb = (Nq + C::BM - 1) / C::BM;
  const int64_t total64 = (int64_t)B * Hq * nqb;
  if (total64 > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  const int total = (int)total64;
  const float c_log2 = scale * 1.44269504088896340736f;
  // Grids that leave most compute units idle (fewer workgroups of 128 rows
  // than half the 256 CUs) take the key-split kernel: 32 rows per workgroup,
  // the keys shared out between its four waves.
  if constexpr (!MODS && !VARLEN && !SPARSE && D <= 128) {
    if (total < kSmallGrid && Nk > eta::SplitCfg<D>::BN) {
      using S = eta::SplitCfg<D>;
      const int nqb32 = (Nq + S::BM - 1) / S::BM;
      const int prescale = !(scale > 0.f) ? 1 : 0;
      hipLaunchKernelGGL((eta::attn_fwd_splitk_kernel<D, BF16, CAUSAL>),
                         dim3((unsigned)((int64_t)B * Hq * nqb32)), dim3(S::kThreads), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, Hq,
                         Hkv, Nq, Nk, nqb32, c_log2, prescale);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
  }
  // d = 256, plain: the 16x16x32 kernel with 32-key tiles, two workgroups
  // of 128 rows per CU.
  if constexpr (!MODS && !VARLEN && !SPARSE && D == 256) {
    if (scale > 0.f) {
      static_assert(eta::K16Cfg<D>::BM == C::BM, "one workgroup per 128-row block");
      hipLaunchKernelGGL((eta::attn_fwd_k16_kernel<D, BF16, CAUSAL>), dim3(total),
                         dim3(eta::K16Cfg<D>::kThreads), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, Hq,
                         Hkv, Nq, Nk, nqb, total, c_log2, eta::VarlenArgs{}, eta::BlockMaskArgs{}, -1,
                         -1);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
  }
  // d = 128 without score variants (plain, packed sequences, block mask):
  // the same tiling on 16x16x32 matrix instructions; non-causal calls
  // without a block mask in workgroups of 256 query rows.  At d = 64 the
  // causal calls only (batched causal measured 3.5-5 % faster, non-causal
  // 8-14 % slower); packed and block-mask causal calls go with them, so that
  // they keep computing bit for bit what the batched causal call computes.
  if constexpr (!MODS && (D == 128 || (D == 64 && CAUSAL))) {
    if (scale > 0.f) {
      if constexpr (!CAUSAL && !SPARSE) {
        using W = eta::K16Cfg<D, true>;
        const int nqbw = (Nq + W::BM - 1) / W::BM;
        const int totalw = (int)((int64_t)B * Hq * nqbw);
        hipLaunchKernelGGL((eta::attn_fwd_k16_kernel<D, BF16, false, VARLEN, false, true>), dim3(totalw),
                           dim3(W::kThreads), 0, stream, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                           static_cast<uint16_t*>(out), lse, Hq, Hkv, Nq, Nk, nqbw, totalw, c_log2, va,
                           bm, -1, -1);
      } else {
        hipLaunchKernelGGL((eta::attn_fwd_k16_kernel<D, BF16, CAUSAL, VARLEN, SPARSE>), dim3(total),
                           dim3(eta::K16Cfg<D>::kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, Hq,
                           Hkv, Nq, Nk, nqb, total, c_log2, va, bm, -1, -1);
      }
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
  }
  // d = 128 with a window alone: the 16x16x32 kernel (128-row workgroups).
  if constexpr (MODS && !VARLEN && !SPARSE && D == 128) {
    if (scale > 0.f && !mods.slopes && !(mods.cap > 0.f)) {
      hipLaunchKernelGGL((eta::attn_fwd_k16_kernel<D, BF16, CAUSAL, false, false, false, true>),
                         dim3(total), dim3(eta::K16Cfg<D>::kThreads), 0, stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, Hq, Hkv, Nq,
                         Nk, nqb, total, c_log2, va, bm, mods.left, mods.right);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
  }
  // Softcap and ALiBi transform the raw scores themselves (no prescaling);
  // a window alone keeps the plain kernel's scaling.
  const bool transform = MODS && (mods.slopes || mods.cap > 0.f);
  const int prescale = (!transform && !(scale > 0.f)) ? 1 : 0;
  hipLaunchKernelGGL((eta::attn_fwd_kernel<D, BF16, CAUSAL, MODS, VARLEN, SPARSE>), dim3(total),
                     dim3(C::kThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<uint16_t*>(out), lse, Hq, Hkv, Nq, Nk, nqb, total, c_log2, prescale,
                     mods, va, bm);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <int D, bool MODS>
int dispatch_dtype(bool bf16, bool causal, const void* q, const void* k, const void* v, void* out,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                   const eta::ScoreMods& m, hipStream_t s) {
  if (bf16) {
    return causal ? launch<D, true, true, MODS>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s)
                  : launch<D, true, false, MODS>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s);
  }
  return causal ? launch<D, false, true, MODS>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s)
                : launch<D, false, false, MODS>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s);
}

template <bool MODS>
int dispatch_hdim(int d, bool bf16, bool c, const void* q, const void* k, const void* v, void* out,
                  float* lse, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                  const eta::ScoreMods& m, hipStream_t s) {
  switch (d) {
    case 64: return dispatch_dtype<64, MODS>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s);
    case 128: return dispatch_dtype<128, MODS>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s);
    default: return dispatch_dtype<256, MODS>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, m, s);
  }
}

// attn_fwd and attn_fwd_ext: validation in the documented order, then the
// plain kernel or, when a score variant is active, its variant instance.
int fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
             const eta::ScoreMods* mods, void* stream) {
  // 1. shape
  if (B < 0 || Nq < 0 || Hq < 1 || Hkv < 1 || Nk < 1 || d < 1) return ATTN_ERR_BAD_SHAPE;
  // 2. empty problem: nothing to do
  if (B == 0 || Nq == 0) return ATTN_OK;
  // Element counts must fit comfortably in 64-bit byte offsets.
  const double q_elems = (double)B * Nq * Hq * d, kv_elems = (double)B * Nk * Hkv * d;
  if (q_elems > 0x1p60 || kv_elems > 0x1p60) return ATTN_ERR_BAD_SHAPE;
  // The kernels address a 128-row window of q/out and a 64-row tile of k/v
  // with 32-bit byte offsets.
  if ((double)128 * Hq * d * 2 >= 0x1p31 || (double)64 * Hkv * d * 2 >= 0x1p31)
    return ATTN_ERR_BAD_SHAPE;
  // The grid holds one workgroup per 128 query rows of every (b, head).
  if ((double)B * Hq * ((Nq + 127) / 128) > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  // 3. null pointers
  if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL_POINTER;
  // 4. GQA ratio
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  // 5. head dimension
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  // 6. element type
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  // 7. scale, and the score variants' arguments
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  if (mods && (mods->left < -1 || mods->right < -1 || !finite_bits(mods->cap) || mods->cap < 0.f))
    return ATTN_ERR_BAD_ARGUMENT;
  // 8. alignment (16-byte vector loads and stores; 4-byte slopes)
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  if (mods && mods->slopes && (reinterpret_cast<uintptr_t>(mods->slopes) & 3)) return ATTN_ERR_MISALIGNED;
  // 9. aliasing: outputs must not overlap inputs or each other
  const size_t qb = (size_t)q_elems * 2, kvb = (size_t)kv_elems * 2;
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb) ||
      overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kvb) || overlaps(lse, lb, v, kvb) ||
      overlaps(out, qb, lse, lb))
    return ATTN_ERR_ALIASING;
  if (mods && mods->slopes &&
      (overlaps(out, qb, mods->slopes, Hq * 4) || overlaps(lse, lb, mods->slopes, Hq * 4)))
    return ATTN_ERR_ALIASING;
  // 10. device
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  // 11. launch
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  const bool c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool active = mods && (mods->left >= 0 || mods->right >= 0 || mods->slopes || mods->cap > 0.f);
  if (active) return dispatch_hdim<true>(d, bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, *mods, s);
  const eta::ScoreMods none{-1, -1, nullptr, 0.f, scale};
  return dispatch_hdim<false>(d, bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, none, s);
}

template <int D>
int dispatch_varlen(bool bf16, bool causal, const void* q, const void* k, const void* v, void* out,
                    float* lse, int B, int Hq, int Hkv, int max_q, float scale,
                    const eta::VarlenArgs& va, hipStream_t s) {
  const eta::ScoreMods none{-1, -1, nullptr, 0.f, scale};
  // Nq = max_q sizes the grid; the kernel reads each sequence's lengths.
  if (bf16) {
    return causal ? launch<D, true, true, false, true>(q, k, v, out, lse, B, Hq, Hkv, max_q, 1, scale, none, s, va)
                  : launch<D, true, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, max_q, 1, scale, none, s, va);
  }
  return causal ? launch<D, false, true, false, true>(q, k, v, out, lse, B, Hq, Hkv, max_q, 1, scale, none, s, va)
                : launch<D, false, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, max_q, 1, scale, none, s, va);
}

template <int D>
int dispatch_sparse(bool bf16, bool causal, const void* q, const void* k, const void* v, void* out,
                    float* lse, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                    const eta::BlockMaskArgs& bm, hipStream_t s) {
  const eta::ScoreMods none{-1, -1, nullptr, 0.f, scale};
  const eta::VarlenArgs nv{nullptr, nullptr, 0, 0, 0};
  if (bf16) {
    return causal ? launch<D, true, true, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, none, s, nv, bm)
                  : launch<D, true, false, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, none, s, nv, bm);
  }
  return causal ? launch<D, false, true, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, none, s, nv, bm)
                : launch<D, false, false, false, false, true>(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, none, s, nv, bm);
}

}  // namespace

extern "C" int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* out,
                                    float* lse, const unsigned char* block_mask, int mask_heads,
                                    int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                                    int causal, int dtype, void* stream) {
  // 1. shape
  if (B < 0 || Nq < 0 || Hq < 1 || Hkv < 1 || Nk < 1 || d < 1) return ATTN_ERR_BAD_SHAPE;
  // 2. empty problem: nothing to do
  if (B == 0 || Nq == 0) return ATTN_OK;
  const double q_elems = (double)B * Nq * Hq * d, kv_elems = (double)B * Nk * Hkv * d;
  if (q_elems > 0x1p60 || kv_elems > 0x1p60) return ATTN_ERR_BAD_SHAPE;
  if ((double)128 * Hq * d * 2 >= 0x1p31 || (double)64 * Hkv * d * 2 >= 0x1p31)
    return ATTN_ERR_BAD_SHAPE;
  if ((double)B * Hq * ((Nq + 127) / 128) > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  const int nqb = (Nq + eta::kMaskBlock - 1) / eta::kMaskBlock;
  const int nkb = (Nk + eta::kMaskBlock - 1) / eta::kMaskBlock;
  // 3. null pointers
  if (!q || !k || !v || !out || !lse || !block_mask) return ATTN_ERR_NULL_POINTER;
  // 4-7. GQA ratio, head dimension, element type, scale, mask heads
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  if (mask_heads != 1 && mask_heads != Hq) return ATTN_ERR_BAD_ARGUMENT;
  // 8. alignment (the mask is read byte by byte)
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  // 9. aliasing: outputs must not overlap the inputs (mask included) or each other
  const size_t qb = (size_t)q_elems * 2, kvb = (size_t)kv_elems * 2;
  const size_t lb = (size_t)B * Hq * Nq * sizeof(float);
  const size_t mb = (size_t)B * mask_heads * nqb * nkb;
  const void* in_p[4] = {q, k, v, block_mask};
  const size_t in_n[4] = {qb, kvb, kvb, mb};
  for (int i = 0; i < 4; ++i)
    if (overlaps(out, qb, in_p[i], in_n[i]) || overlaps(lse, lb, in_p[i], in_n[i])) return ATTN_ERR_ALIASING;
  if (overlaps(out, qb, lse, lb)) return ATTN_ERR_ALIASING;
  // 10. device
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  // 11. launch
  const eta::BlockMaskArgs bm{block_mask, mask_heads, nkb};
  const bool bf16 = dtype == ATTN_DTYPE_BF16, c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 64: return dispatch_sparse<64>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, bm, s);
    case 128: return dispatch_sparse<128>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, bm, s);
    default: return dispatch_sparse<256>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, scale, bm, s);
  }
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                               const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                               int Hkv, int total_q, int total_k, int max_seqlen_q, int d,
                               float scale, int causal, int dtype, void* stream) {
  // 1. shape
  if (B < 0 || Hq < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || d < 1)
    return ATTN_ERR_BAD_SHAPE;
  // 2. nothing to do
  if (B == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
  const double q_elems = (double)total_q * Hq * d, kv_elems = (double)total_k * Hkv * d;
  if (q_elems > 0x1p60 || kv_elems > 0x1p60) return ATTN_ERR_BAD_SHAPE;
  if ((double)128 * Hq * d * 2 >= 0x1p31 || (double)64 * Hkv * d * 2 >= 0x1p31)
    return ATTN_ERR_BAD_SHAPE;
  if ((double)B * Hq * ((max_seqlen_q + 127) / 128) > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  // 3. null pointers (k and v may be NULL only when there are no keys)
  if (!q || !out || !lse || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_POINTER;
  if (total_k > 0 && (!k || !v)) return ATTN_ERR_NULL_POINTER;
  // 4-7. GQA ratio, head dim, dtype, scale
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  // 8. alignment
  if (!aligned16(q) || !aligned16(out) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3))
    return ATTN_ERR_MISALIGNED;
  if (total_k > 0 && (!aligned16(k) || !aligned16(v))) return ATTN_ERR_MISALIGNED;
  // 9. aliasing: outputs must not overlap the inputs or each other
  const size_t qb = (size_t)q_elems * 2, kvb = (size_t)kv_elems * 2;
  const size_t lb = (size_t)Hq * total_q * sizeof(float), cb = (size_t)(B + 1) * 4;
  const void* in_p[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const size_t in_n[5] = {qb, kvb, kvb, cb, cb};
  for (int i = 0; i < 5; ++i) {
    if (!in_p[i] || !in_n[i]) continue;
    if (overlaps(out, qb, in_p[i], in_n[i]) || overlaps(lse, lb, in_p[i], in_n[i])) return ATTN_ERR_ALIASING;
  }
  if (overlaps(out, qb, lse, lb)) return ATTN_ERR_ALIASING;
  // 10. device
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  // 11. launch
  const eta::VarlenArgs va{cu_seqlens_q, cu_seqlens_k, total_q, total_k, B * Hq};
  const bool bf16 = dtype == ATTN_DTYPE_BF16, c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 64: return dispatch_varlen<64>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, max_seqlen_q, scale, va, s);
    case 128: return dispatch_varlen<128>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, max_seqlen_q, scale, va, s);
    default: return dispatch_varlen<256>(bf16, c, q, k, v, out, lse, B, Hq, Hkv, max_seqlen_q, scale, va, s);
  }
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                        int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                        void* stream) {
  return fwd_impl(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, nullptr, stream);
}

extern "C" int attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                            int window_left, int window_right, const float* alibi_slopes,
                            float softcap, int dtype, void* stream) {
  const eta::ScoreMods mods{window_left, window_right, alibi_slopes, softcap, scale};
  return fwd_impl(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, &mods, stream);
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_NULL_POINTER: return "ATTN_ERR_NULL_POINTER: q, k, v, out or lse is NULL";
    case ATTN_ERR_BAD_SHAPE:
      return "ATTN_ERR_BAD_SHAPE: need B>=0, Nq>=0, Hq>=1, Hkv>=1, Nk>=1, d>=1 and a size that fits";
    case ATTN_ERR_GQA_RATIO: return "ATTN_ERR_GQA_RATIO: Hq must be a multiple of Hkv";
    case ATTN_ERR_UNSUPPORTED_HDIM: return "ATTN_ERR_UNSUPPORTED_HDIM: d must be 64, 128 or 256";
    case ATTN_ERR_UNSUPPORTED_DTYPE: return "ATTN_ERR_UNSUPPORTED_DTYPE: dtype must be fp16 or bf16";
    case ATTN_ERR_BAD_SCALE: return "ATTN_ERR_BAD_SCALE: scale must be finite";
    case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED: every pointer must be 16-byte aligned";
    case ATTN_ERR_ALIASING: return "ATTN_ERR_ALIASING: out and lse must not overlap the inputs or each other";
    case ATTN_ERR_NO_DEVICE: return "ATTN_ERR_NO_DEVICE: no HIP device, or the current device is not gfx950";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: kernel launch failed";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace smaller than attn_decode_workspace_size";
    case ATTN_ERR_BAD_ARGUMENT:
      return "ATTN_ERR_BAD_ARGUMENT: window bounds must be >= -1, softcap finite and >= 0, "
             "mask_heads 1 or Hq";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "ATTN_ERR_SCRATCH_LIMIT: the split partials exceed the 8 MiB scratch of "
             "attn_decode_noalloc; use fewer splits, or attn_decode with a workspace";
    default: return "unknown attn status";
  }
}

extern "C" const char* attn_version(void) { return kVersion; }
