// C ABI of the exact tiled attention backward (declared in include/attn.h).
//
// Host side only: argument validation before any HIP call, the cached gfx950
// check, and two asynchronous launches on the caller's stream: the dQ kernel
// (which also writes delta) and then the dK/dV kernel (which reads it).
// No device memory is allocated.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.h"
#include "attn_bwd_kernel.hpp"
#include "attn_host.hpp"

namespace {

using eta_host::aligned16;
using eta_host::check_device;
using eta_host::finite_bits;
using eta_host::overlaps;

template <int D, bool BF16, bool CAUSAL, bool SPARSE, int MK = 0>
int launch_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq,
               int Hkv, int Nq, int Nk, float scale, const eta::BlockMaskArgs& bm,
               hipStream_t stream, const eta::ScoreMods& mods) {
  using CQ = eta::DqCfg<D>;
  using CK = eta::DkvCfg<D>;
  const float c_log2 = scale * eta::kLog2e;
  const int nqb = (Nq + CQ::BM - 1) / CQ::BM;
  const int nkb = (Nk + CK::BK - 1) / CK::BK;
  const int64_t tq = (int64_t)B * Hq * nqb, tk = (int64_t)B * Hkv * nkb;
  if (tq > 0x7fffffff || tk > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* Kp = static_cast<const uint16_t*>(k);
  const auto* Vp = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  if (tq > 0) {
    hipLaunchKernelGGL((eta::attn_bwd_dq_kernel<D, BF16, CAUSAL, SPARSE, false, MK>), dim3((int)tq),
                       dim3(CQ::kThreads), 0, stream, Q, Kp, Vp, static_cast<const uint16_t*>(out),
                       dO, lse, static_cast<uint16_t*>(dq), delta, Hq, Hkv, Nq, Nk, nqb, (int)tq,
                       scale, c_log2, bm, eta::VarlenArgs{nullptr, nullptr, 0, 0, 0}, mods);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  // The plain non-causal d = 128 dK/dV kernel runs 256 keys (8 waves) per
  // workgroup.
  if constexpr (!CAUSAL && !SPARSE && MK == 0 && D == 128) {
    using CW = eta::DkvCfg<D, true>;
    const int nkbw = (Nk + CW::BK - 1) / CW::BK;
    const int tkw = (int)((int64_t)B * Hkv * nkbw);
    hipLaunchKernelGGL((eta::attn_bwd_dkdv_kernel<D, BF16, false, false, false, 0, true>), dim3(tkw),
                       dim3(CW::kThreads), 0, stream, Q, Kp, Vp, dO, lse, delta,
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), Hq, Hkv, Nq, Nk, nkbw,
                       tkw, scale, c_log2, bm, eta::VarlenArgs{nullptr, nullptr, 0, 0, 0}, mods);
  } else {
    hipLaunchKernelGGL((eta::attn_bwd_dkdv_kernel<D, BF16, CAUSAL, SPARSE, false, MK>), dim3((int)tk),
                       dim3(CK::kThreads), 0, stream, Q, Kp, Vp, dO, lse, delta,
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), Hq, Hkv, Nq, Nk, nkb,
                       (int)tk, scale, c_log2, bm, eta::VarlenArgs{nullptr, nullptr, 0, 0, 0}, mods);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Packed sequences: one dQ workgroup per (sequence, query head, 128 query
// rows of the longest query sequence), one dK/dV workgroup per (sequence,
// KV head, 128 keys of the longest key sequence); workgroups past their
// sequence's end exit at once.
template <int D, bool BF16, bool CAUSAL>
int launch_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, const int* cu_q, const int* cu_k, int B, int Hq, int Hkv,
                      int total_q, int total_k, int max_q, int max_k, float scale,
                      hipStream_t stream) {
  using CQ = eta::DqCfg<D>;
  using CK = eta::DkvCfg<D>;
  const float c_log2 = scale * eta::kLog2e;
  const int nqb = (max_q + CQ::BM - 1) / CQ::BM;
  const int nkb = (max_k + CK::BK - 1) / CK::BK;
  const int64_t tq = (int64_t)B * Hq * nqb, tk = (int64_t)B * Hkv * nkb;
  if (tq > 0x7fffffff || tk > 0x7fffffff) return ATTN_ERR_BAD_SHAPE;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* Kp = static_cast<const uint16_t*>(k);
  const auto* Vp = static_cast<const uint16_t*>(v);
  const auto* dO = static_cast<const uint16_t*>(dout);
  const eta::BlockMaskArgs nb{nullptr, 1, 0};
  if (tq > 0) {
    const eta::VarlenArgs va{cu_q, cu_k, total_q, total_k, B * Hq};
    hipLaunchKernelGGL((eta::attn_bwd_dq_kernel<D, BF16, CAUSAL, false, true>), dim3((int)tq),
                       dim3(CQ::kThreads), 0, stream, Q, Kp, Vp, static_cast<const uint16_t*>(out),
                       dO, lse, static_cast<uint16_t*>(dq), delta, Hq, Hkv, max_q, max_k, nqb,
                       (int)tq, scale, c_log2, nb, va, eta::ScoreMods{-1, -1, nullptr, 0.f, scale});
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  if (tk > 0) {
    const eta::VarlenArgs va{cu_q, cu_k, total_q, total_k, B * Hkv};
    hipLaunchKernelGGL((eta::attn_bwd_dkdv_kernel<D, BF16, CAUSAL, false, true>), dim3((int)tk),
                       dim3(CK::kThreads), 0, stream, Q, Kp, Vp, dO, lse, delta,
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), Hq, Hkv, max_q,
                       max_k, nkb, (int)tk, scale, c_log2, nb, va,
                       eta::ScoreMods{-1, -1, nullptr, 0.f, scale});
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

template <int D, bool SPARSE, int MK>
int dispatch_bwd(bool bf16, bool causal, const void* q, const void* k, const void* v,
                 const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 float* delta, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                 const eta::BlockMaskArgs& bm, hipStream_t s, const eta::ScoreMods& m) {
#define ETA_BWD_ARGS q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, m
  if (bf16) {
    return causal ? launch_bwd<D, true, true, SPARSE, MK>(ETA_BWD_ARGS)
                  : launch_bwd<D, true, false, SPARSE, MK>(ETA_BWD_ARGS);
  }
  return causal ? launch_bwd<D, false, true, SPARSE, MK>(ETA_BWD_ARGS)
                : launch_bwd<D, false, false, SPARSE, MK>(ETA_BWD_ARGS);
#undef ETA_BWD_ARGS
}

template <bool SPARSE, int MK = 0>
int dispatch_hdim(int d, bool bf16, bool c, const void* q, const void* k, const void* v,
                  const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  float* delta, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                  const eta::BlockMaskArgs& bm, hipStream_t s, const eta::ScoreMods& m) {
  switch (d) {
    case 64:
      return dispatch_bwd<64, SPARSE, MK>(bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, m);
    case 128:
      return dispatch_bwd<128, SPARSE, MK>(bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, m);
    default:
      return dispatch_bwd<256, SPARSE, MK>(bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, m);
  }
}

// attn_bwd and attn_bwd_blocksparse: validation in the documented order,
// then the plain kernels or (with a block mask) their block-sparse instances.
int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             const unsigned char* block_mask, int mask_heads, bool sparse, int B, int Hq, int Hkv,
             int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream,
             const eta::ScoreMods* mods = nullptr) {
  // 1. shape
  if (B < 0 || Nq < 0 || Hq < 1 || Hkv < 1 || Nk < 1 || d < 1) return ATTN_ERR_BAD_SHAPE;
  // 2. empty batch: nothing to do
  if (B == 0) return ATTN_OK;
  const double q_elems = (double)B * Nq * Hq * d, kv_elems = (double)B * Nk * Hkv * d;
  if (q_elems > 0x1p60 || kv_elems > 0x1p60) return ATTN_ERR_BAD_SHAPE;
  // The kernels address 128-row windows of q-shaped and k-shaped tensors
  // with 32-bit byte offsets, and grids of one workgroup per 128 rows.
  if ((double)128 * Hq * d * 2 >= 0x1p31 || (double)128 * Hkv * d * 2 >= 0x1p31)
    return ATTN_ERR_BAD_SHAPE;
  if ((double)B * Hq * ((Nq + 127) / 128) > 0x7fffffff ||
      (double)B * Hkv * ((Nk + 127) / 128) > 0x7fffffff)
    return ATTN_ERR_BAD_SHAPE;
  // 3. null pointers (with Nq == 0 only k, v, dk and dv are touched)
  if (!k || !v || !dk || !dv) return ATTN_ERR_NULL_POINTER;
  const bool rows = Nq > 0;
  if (rows && (!q || !out || !dout || !lse || !dq || !delta)) return ATTN_ERR_NULL_POINTER;
  if (sparse && rows && !block_mask) return ATTN_ERR_NULL_POINTER;
  // 4. GQA ratio, 5. head dimension, 6. element type, 7. scale
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  if (sparse && mask_heads != 1 && mask_heads != Hq) return ATTN_ERR_BAD_ARGUMENT;
  if (mods && (mods->left < -1 || mods->right < -1 || !finite_bits(mods->cap) || mods->cap < 0.f))
    return ATTN_ERR_BAD_ARGUMENT;
  // 8. alignment
  if (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_MISALIGNED;
  if (rows && (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(lse) ||
               !aligned16(dq) || !aligned16(delta)))
    return ATTN_ERR_MISALIGNED;
  if (rows && mods && mods->slopes && (reinterpret_cast<uintptr_t>(mods->slopes) & 3))
    return ATTN_ERR_MISALIGNED;
  // 9. aliasing: no output overlaps an input or another output
  const size_t qb = rows ? (size_t)q_elems * 2 : 0, kvb = (size_t)kv_elems * 2;
  const size_t vb = rows ? (size_t)B * Hq * Nq * sizeof(float) : 0;
  const int nqbm = (Nq + eta::kMaskBlock - 1) / eta::kMaskBlock;
  const int nkbm = (Nk + eta::kMaskBlock - 1) / eta::kMaskBlock;
  const size_t mb = sparse && rows ? (size_t)B * mask_heads * nqbm * nkbm : 0;
  const size_t sb = rows && mods && mods->slopes ? (size_t)Hq * 4 : 0;
  const void* in_p[8] = {q, k, v, out, dout, lse, block_mask, mods ? mods->slopes : nullptr};
  const size_t in_n[8] = {qb, kvb, kvb, qb, qb, vb, mb, sb};
  const void* out_p[4] = {dq, dk, dv, delta};
  const size_t out_n[4] = {qb, kvb, kvb, vb};
  for (int i = 0; i < 4; ++i) {
    if (out_n[i] == 0) continue;
    for (int j = 0; j < 8; ++j)
      if (in_n[j] && overlaps(out_p[i], out_n[i], in_p[j], in_n[j])) return ATTN_ERR_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (out_n[j] && overlaps(out_p[i], out_n[i], out_p[j], out_n[j])) return ATTN_ERR_ALIASING;
  }
  // 10. device
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  // 11. launch
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  const bool c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const eta::BlockMaskArgs bm{sparse && rows ? block_mask : nullptr, sparse ? mask_heads : 1, nkbm};
  const bool active = mods && (mods->left >= 0 || mods->right >= 0 || mods->slopes || mods->cap > 0.f);
  const eta::ScoreMods none{-1, -1, nullptr, 0.f, scale};
  if (sparse)
    return dispatch_hdim<true>(d, bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, none);
  if (active) {
#define ETA_MODS_ARGS d, bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, *mods
    using eta::kModsAlibi;
    using eta::kModsCap;
    using eta::kModsOn;
    // One instance per combination of softcap and ALiBi (the window is read
    // at run time by all four).
    const bool cap = mods->cap > 0.f, alibi = mods->slopes != nullptr;
    if (cap && alibi) return dispatch_hdim<false, kModsOn | kModsCap | kModsAlibi>(ETA_MODS_ARGS);
    if (cap) return dispatch_hdim<false, kModsOn | kModsCap>(ETA_MODS_ARGS);
    if (alibi) return dispatch_hdim<false, kModsOn | kModsAlibi>(ETA_MODS_ARGS);
    return dispatch_hdim<false, kModsOn>(ETA_MODS_ARGS);
#undef ETA_MODS_ARGS
  }
  return dispatch_hdim<false>(d, bf16, c, q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nk, scale, bm, s, none);
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        int causal, int dtype, void* stream) {
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, delta, nullptr, 1, false, B, Hq, Hkv, Nq, Nk,
                  d, scale, causal, dtype, stream);
}

extern "C" int attn_bwd_ext(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* delta, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                            int causal, int window_left, int window_right,
                            const float* alibi_slopes, float softcap, int dtype, void* stream) {
  const eta::ScoreMods mods{window_left, window_right, alibi_slopes, softcap, scale};
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, delta, nullptr, 1, false, B, Hq, Hkv, Nq, Nk,
                  d, scale, causal, dtype, stream, &mods);
}

extern "C" int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out,
                                    const void* dout, const float* lse, void* dq, void* dk,
                                    void* dv, float* delta, const unsigned char* block_mask,
                                    int mask_heads, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                    float scale, int causal, int dtype, void* stream) {
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, delta, block_mask, mask_heads, true, B, Hq,
                  Hkv, Nq, Nk, d, scale, causal, dtype, stream);
}

extern "C" int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               float* delta, const int* cu_seqlens_q, const int* cu_seqlens_k,
                               int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                               int max_seqlen_k, int d, float scale, int causal, int dtype,
                               void* stream) {
  // 1. shape
  if (B < 0 || Hq < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 ||
      max_seqlen_k < 0 || d < 1)
    return ATTN_ERR_BAD_SHAPE;
  // 2. nothing to do
  if (B == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
  const double q_elems = (double)total_q * Hq * d, kv_elems = (double)total_k * Hkv * d;
  if (q_elems > 0x1p60 || kv_elems > 0x1p60) return ATTN_ERR_BAD_SHAPE;
  if ((double)128 * Hq * d * 2 >= 0x1p31 || (double)128 * Hkv * d * 2 >= 0x1p31)
    return ATTN_ERR_BAD_SHAPE;
  if ((double)B * Hq * ((max_seqlen_q + 127) / 128) > 0x7fffffff ||
      (double)B * Hkv * ((max_seqlen_k + 127) / 128) > 0x7fffffff)
    return ATTN_ERR_BAD_SHAPE;
  // 3. null pointers: the row buffers of whichever side has rows
  const bool qrows = total_q > 0, krows = total_k > 0;
  if (!cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_POINTER;
  if (qrows && (!q || !out || !dout || !lse || !dq || !delta)) return ATTN_ERR_NULL_POINTER;
  if (krows && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL_POINTER;
  // 4-7. GQA ratio, head dimension, element type, scale
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  // 8. alignment
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3))
    return ATTN_ERR_MISALIGNED;
  if (qrows && (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(lse) ||
                !aligned16(dq) || !aligned16(delta)))
    return ATTN_ERR_MISALIGNED;
  if (krows && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv)))
    return ATTN_ERR_MISALIGNED;
  // 9. aliasing: no output overlaps an input or another output
  const size_t qb = (size_t)q_elems * 2, kvb = (size_t)kv_elems * 2;
  const size_t vb = (size_t)Hq * total_q * sizeof(float), cb = (size_t)(B + 1) * 4;
  const void* in_p[8] = {q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k};
  const size_t in_n[8] = {qb, kvb, kvb, qb, qb, vb, cb, cb};
  const void* out_p[4] = {dq, dk, dv, delta};
  const size_t out_n[4] = {qb, kvb, kvb, vb};
  for (int i = 0; i < 4; ++i) {
    if (out_n[i] == 0 || !out_p[i]) continue;
    for (int j = 0; j < 8; ++j)
      if (in_n[j] && in_p[j] && overlaps(out_p[i], out_n[i], in_p[j], in_n[j])) return ATTN_ERR_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (out_n[j] && out_p[j] && overlaps(out_p[i], out_n[i], out_p[j], out_n[j]))
        return ATTN_ERR_ALIASING;
  }
  // 10. device
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  // 11. launch (a side without rows launches nothing)
  const bool bf16 = dtype == ATTN_DTYPE_BF16, c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mq = qrows ? max_seqlen_q : 0, mk = krows ? max_seqlen_k : 0;
#define ETA_VL_ARGS q, k, v, out, dout, lse, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k, mq, mk, scale, s
  switch (d) {
    case 64:
      return bf16 ? (c ? launch_bwd_varlen<64, true, true>(ETA_VL_ARGS) : launch_bwd_varlen<64, true, false>(ETA_VL_ARGS))
                  : (c ? launch_bwd_varlen<64, false, true>(ETA_VL_ARGS) : launch_bwd_varlen<64, false, false>(ETA_VL_ARGS));
    case 128:
      return bf16 ? (c ? launch_bwd_varlen<128, true, true>(ETA_VL_ARGS) : launch_bwd_varlen<128, true, false>(ETA_VL_ARGS))
                  : (c ? launch_bwd_varlen<128, false, true>(ETA_VL_ARGS) : launch_bwd_varlen<128, false, false>(ETA_VL_ARGS));
    default:
      return bf16 ? (c ? launch_bwd_varlen<256, true, true>(ETA_VL_ARGS) : launch_bwd_varlen<256, true, false>(ETA_VL_ARGS))
                  : (c ? launch_bwd_varlen<256, false, true>(ETA_VL_ARGS) : launch_bwd_varlen<256, false, false>(ETA_VL_ARGS));
  }
#undef ETA_VL_ARGS
}
