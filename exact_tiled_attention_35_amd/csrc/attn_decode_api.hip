// C ABI of the KV-cache decode forward (declared in include/attn.h).
//
// Host side only: validation before any HIP call, the split heuristic, the
// workspace size, and up to three asynchronous launches on the caller's
// stream (cache append, split attention, merge).  No device memory is
// allocated: the split partials live in the caller's workspace, or, for
// attn_decode_noalloc, in the library's own scratch array.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "attn_decode_kernel.hpp"
#include "attn_host.hpp"

// Scratch of attn_decode_noalloc: the split partials, one array per GPU the
// library runs on, held until the process ends.  In host code the array's
// name is only a stand-in; the address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to the kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

using eta_host::aligned16;
using eta_host::check_device;
using eta_host::finite_bits;
using eta_host::overlaps;

constexpr int kMaxSplits = 128;
constexpr int kTargetWorkgroups = 512;  // two per CU on MI355X's 256 CUs

int row_blocks(int Hq, int Hkv, int Nq) { return (Hq / Hkv * Nq + 127) / 128; }

size_t part_o_bytes(int B, int Hq, int Nq, int d, int splits) {
  return (size_t)splits * B * Hq * Nq * d * sizeof(float);
}

template <int D, bool BF16, bool CAUSAL>
int launch_decode(const void* q, void* kc, void* vc, const int* seqlens, const void* kn,
                  const void* vn, void* out, float* lse, void* ws, int B, int Hq, int Hkv,
                  int Nq, int Ncap, int Nnew, float scale, int splits, hipStream_t s) {
  auto* K = static_cast<uint16_t*>(kc);
  auto* V = static_cast<uint16_t*>(vc);
  // With query rows the attention kernel appends the new rows itself; a
  // call without query rows only appends.
  if (Nq == 0) {
    if (Nnew > 0) {
      const int64_t n = (int64_t)B * Nnew * Hkv * (D / 8);
      hipLaunchKernelGGL((eta::kv_append_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                         0, s, static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn), K,
                         V, seqlens, B, Nnew, Hkv, Ncap);
      if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
    }
    return ATTN_OK;
  }
  const int nrb = row_blocks(Hq, Hkv, Nq);
  const int64_t grid = (int64_t)B * Hkv * nrb * splits;
  float* opart = splits > 1 ? static_cast<float*>(ws) : nullptr;
  float* lpart = splits > 1
                     ? reinterpret_cast<float*>(static_cast<char*>(ws) + part_o_bytes(B, Hq, Nq, D, splits))
                     : nullptr;
  const float c_log2 = scale * 1.44269504088896340736f;
  hipLaunchKernelGGL((eta::attn_decode_kernel<D, BF16, CAUSAL>), dim3((unsigned)grid),
                     dim3(eta::DecCfg<D>::kThreads), 0, s, static_cast<const uint16_t*>(q), K, V,
                     seqlens, static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn),
                     static_cast<uint16_t*>(out), lse, opart, lpart, B, Hq, Hkv, Nq, Ncap,
                     Nnew, nrb, splits, c_log2, scale > 0.f ? 0 : 1);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  if (splits > 1) {
    const int64_t rows = (int64_t)B * Hq * Nq;
    hipLaunchKernelGGL((eta::attn_decode_merge_kernel<D, BF16>), dim3((unsigned)((rows + 3) / 4)),
                       dim3(256), 0, s, opart, lpart, static_cast<uint16_t*>(out), lse, B, Hq, Nq,
                       splits);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

template <int D>
int dispatch_decode(bool bf16, bool causal, const void* q, void* kc, void* vc, const int* sl,
                    const void* kn, const void* vn, void* out, float* lse, void* ws, int B,
                    int Hq, int Hkv, int Nq, int Ncap, int Nnew, float scale, int splits,
                    hipStream_t s) {
#define ETA_DEC_ARGS q, kc, vc, sl, kn, vn, out, lse, ws, B, Hq, Hkv, Nq, Ncap, Nnew, scale, splits, s
  if (bf16)
    return causal ? launch_decode<D, true, true>(ETA_DEC_ARGS) : launch_decode<D, true, false>(ETA_DEC_ARGS);
  return causal ? launch_decode<D, false, true>(ETA_DEC_ARGS) : launch_decode<D, false, false>(ETA_DEC_ARGS);
#undef ETA_DEC_ARGS
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return ATTN_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();  // do not leave the error for the caller's next call
      return ATTN_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

int decode_impl(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                const void* k_new, const void* v_new, void* out, float* lse, void* workspace,
                size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Ncap, int Nnew, int d,
                float scale, int causal, int dtype, int num_splits, void* stream, bool use_scratch);

}  // namespace

extern "C" int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Ncap, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Ncap < 1 || d < 1 || Hq % Hkv != 0) return 1;
  const int64_t wgs = (int64_t)B * Hkv * row_blocks(Hq, Hkv, Nq);
  int64_t splits = (kTargetWorkgroups + wgs - 1) / wgs;
  // At least four 32-key tiles per split.
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, Ncap / 128));
  return (int)std::max<int64_t>(1, std::min<int64_t>(splits, kMaxSplits));
}

extern "C" size_t attn_decode_workspace_size(int B, int Hq, int Nq, int d, int num_splits) {
  if (num_splits <= 1 || B < 1 || Hq < 1 || Nq < 1 || d < 1) return 0;
  return part_o_bytes(B, Hq, Nq, d, num_splits) + (size_t)num_splits * B * Hq * Nq * sizeof(float);
}

extern "C" int attn_decode(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                           const void* k_new, const void* v_new, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                           int Ncap, int Nnew, int d, float scale, int causal, int dtype,
                           int num_splits, void* stream) {
  return decode_impl(q, k_cache, v_cache, cache_seqlens, k_new, v_new, out, lse, workspace,
                     workspace_bytes, B, Hq, Hkv, Nq, Ncap, Nnew, d, scale, causal, dtype,
                     num_splits, stream, false);
}

extern "C" int attn_decode_noalloc(const void* q, void* k_cache, void* v_cache,
                                   const int* cache_seqlens, const void* k_new, const void* v_new,
                                   void* out, float* lse, int B, int Hq, int Hkv, int Nq, int Ncap,
                                   int Nnew, int d, float scale, int causal, int dtype,
                                   int num_splits, void* stream) {
  return decode_impl(q, k_cache, v_cache, cache_seqlens, k_new, v_new, out, lse, nullptr,
                     ATTN_DECODE_SCRATCH_BYTES, B, Hq, Hkv, Nq, Ncap, Nnew, d, scale, causal,
                     dtype, num_splits, stream, true);
}

namespace {

int decode_impl(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                const void* k_new, const void* v_new, void* out, float* lse, void* workspace,
                size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Ncap, int Nnew, int d,
                float scale, int causal, int dtype, int num_splits, void* stream,
                bool use_scratch) {
  // 1. shape
  if (B < 0 || Nq < 0 || Hq < 1 || Hkv < 1 || Ncap < 1 || Nnew < 0 || Nnew > Ncap || d < 1)
    return ATTN_ERR_BAD_SHAPE;
  // 2. nothing to do
  if (B == 0 || (Nq == 0 && Nnew == 0)) return ATTN_OK;
  const double cache_elems = (double)B * Ncap * Hkv * d;
  if ((double)Ncap * Hkv * d * 2 >= 0x1p31 || (double)Nq * Hq * d * 2 >= 0x1p31 ||
      (double)B * Nnew * Hkv * d * 2 >= 0x1p31 || cache_elems > 0x1p60)
    return ATTN_ERR_BAD_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_BAD_SHAPE;
  int splits = Nq == 0 ? 1 : (num_splits == 0 ? attn_decode_num_splits(B, Hq, Hkv, Nq, Ncap, d) : num_splits);
  if (use_scratch && num_splits == 0 && splits > 1) {
    // the heuristic's count, lowered to what the scratch array holds
    const size_t per_split = attn_decode_workspace_size(B, Hq, Nq, d, 2) / 2;
    splits = (int)std::max<size_t>(1, std::min<size_t>(splits, ATTN_DECODE_SCRATCH_BYTES / per_split));
  }
  if (Hq % Hkv == 0 && (double)B * Hkv * row_blocks(Hq, Hkv, Nq) * splits > 0x7fffffff)
    return ATTN_ERR_BAD_SHAPE;
  // 3. null pointers
  if (!k_cache || !v_cache || !cache_seqlens) return ATTN_ERR_NULL_POINTER;
  if (Nnew > 0 && (!k_new || !v_new)) return ATTN_ERR_NULL_POINTER;
  if (Nq > 0 && (!q || !out || !lse)) return ATTN_ERR_NULL_POINTER;
  if (Nq > 0 && splits > 1 && !workspace && !use_scratch) return ATTN_ERR_NULL_POINTER;
  // 4-7. GQA ratio, head dim, dtype, scale
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_RATIO;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED_HDIM;
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
  if (!finite_bits(scale)) return ATTN_ERR_BAD_SCALE;
  // 8. workspace size and alignment
  const size_t ws_need = Nq > 0 ? attn_decode_workspace_size(B, Hq, Nq, d, splits) : 0;
  if (workspace_bytes < ws_need) return use_scratch ? ATTN_ERR_SCRATCH_LIMIT : ATTN_ERR_WORKSPACE;
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(cache_seqlens) & 3))
    return ATTN_ERR_MISALIGNED;
  if (Nnew > 0 && (!aligned16(k_new) || !aligned16(v_new))) return ATTN_ERR_MISALIGNED;
  if (Nq > 0 && (!aligned16(q) || !aligned16(out) || !aligned16(lse))) return ATTN_ERR_MISALIGNED;
  if (ws_need > 0 && !use_scratch && !aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  // 9. aliasing: written buffers (caches, out, lse, workspace) must not
  // overlap each other or the buffers that are only read
  const size_t cb = (size_t)cache_elems * 2, qb = (size_t)B * Nq * Hq * d * 2;
  const size_t nb = (size_t)B * Nnew * Hkv * d * 2, lb = (size_t)B * Hq * Nq * 4, sb = (size_t)B * 4;
  // (the library's scratch array cannot overlap the caller's buffers)
  const void* wp[5] = {k_cache, v_cache, out, lse, workspace};
  const size_t wn[5] = {cb, cb, qb, lb, use_scratch ? 0 : ws_need};
  const void* rp[4] = {q, cache_seqlens, k_new, v_new};
  const size_t rn[4] = {qb, sb, nb, nb};
  for (int a = 0; a < 5; ++a) {
    if (wn[a] == 0) continue;
    for (int c = 0; c < 4; ++c)
      if (rn[c] && overlaps(wp[a], wn[a], rp[c], rn[c])) return ATTN_ERR_ALIASING;
    for (int c = a + 1; c < 5; ++c)
      if (wn[c] && overlaps(wp[a], wn[a], wp[c], wn[c])) return ATTN_ERR_ALIASING;
  }
  // 10. device (and, for attn_decode_noalloc, the scratch array's address on it)
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;
  if (use_scratch) {
    workspace = nullptr;
    if (ws_need > 0) {
      const int st = scratch_address(&workspace);
      if (st != ATTN_OK) return st;
    }
  }
  // 11. launch
  const bool bf16 = dtype == ATTN_DTYPE_BF16, c = causal != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 64:
      return dispatch_decode<64>(bf16, c, q, k_cache, v_cache, cache_seqlens, k_new, v_new, out, lse, workspace, B, Hq, Hkv, Nq, Ncap, Nnew, scale, splits, s);
    case 128:
      return dispatch_decode<128>(bf16, c, q, k_cache, v_cache, cache_seqlens, k_new, v_new, out, lse, workspace, B, Hq, Hkv, Nq, Ncap, Nnew, scale, splits, s);
    default:
      return dispatch_decode<256>(bf16, c, q, k_cache, v_cache, cache_seqlens, k_new, v_new, out, lse, workspace, B, Hq, Hkv, Nq, Ncap, Nnew, scale, splits, s);
  }
}

}  // namespace
