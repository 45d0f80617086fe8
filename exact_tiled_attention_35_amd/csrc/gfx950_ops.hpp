// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the 32x32x16 MFMA, element packing, raw buffer
// descriptors (loads, stores, direct global->LDS loads), the LDS
// transpose read and the workgroup-to-work-item map.
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

// D = A B + C with A 16x32, B 32x16 (v_mfma_f32_16x16x32_{bf16,f16}): lane l
// holds A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] for e = 0..7,
// and D[4 (l / 16) + r][l % 16] for r = 0..3.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
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

__device__ __forceinline__ void buf_store16(u32x4_t v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

__device__ __forceinline__ void buf_store4(float v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, 0, 0);
}

// Direct global->LDS load: each lane's 16 bytes land at lds_dst + 16 * lane.
__device__ __forceinline__ void buf_load_lds16(rsrc_t r, uint16_t* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane
// group, lane 4a+b receives element b of the 4-element rows addressed by
// lanes a, a+4, a+8, a+12.  With lane i addressing row (i/4) at column
// 4*(i%4) of a row-major [key][d] block, lane i receives 4 consecutive keys
// at column i: one quarter of a 32x32x16 A operand of V^T.
__device__ __forceinline__ u32x2_t lds_read_tr4(const uint16_t* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p));
}

// Score variants (the sliding window, ALiBi and softcapping of the pages'
// interface and version history): with diag = Nk - Nq, key j is kept for row
// i iff i + diag - left <= j <= i + diag + right (negative = no bound); the
// scaled score t becomes cap * tanh(t / cap) when cap > 0, and then
// t - slope[h] * |i + diag - j| when slopes is not NULL.
struct ScoreMods {
  int left, right;
  const float* slopes;
  float cap, sigma;
};

// tanh(x) = 1 - 2 / (2^(2x log2 e) + 1); saturates to +-1 for large |x|.
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_fast(x * 2.88539008177792681472f) + 1.0f);
}

// Variable-length sequences packed along the row axis: sequence b owns
// query rows [cu_q[b], cu_q[b+1]) of q/out and key rows [cu_k[b], cu_k[b+1])
// of k/v; lse (and the backward's delta) is [Hq, total_q].  Offsets are
// clamped to [0, total] so that no access leaves the packed tensors.
struct VarlenArgs {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int pairs;  // sequences x heads of the grid's head axis
};

// Block sparsity: flags over (query block, key block) pairs of 128 x 128
// decide which blocks of the score matrix take part; key j is visible to row
// i only if the flag of (i / 128, j / 128) is nonzero (and causally, when
// causal).  mask is [B, heads, ceil(Nq / 128), nkb] bytes with heads = 1
// (shared by all query heads) or Hq; nkb = ceil(Nk / 128).
constexpr int kMaskBlock = 128;
struct BlockMaskArgs {
  const uint8_t* mask;
  int heads, nkb;
};

// 64 flags of one line of the mask (a row of key blocks, stride 1 byte, or
// a column of query blocks, stride nkb bytes) as one wave-uniform word: lane
// i loads flag 64 c + i through a descriptor whose range ends after the
// line's last flag (flags past it read as 0), and a ballot gathers them.
__device__ __forceinline__ uint64_t flag_word(rsrc_t r, int c, int stride, int lane) {
  return __builtin_amdgcn_ballot_w64(
      __builtin_amdgcn_raw_buffer_load_b8(r, (64 * c + lane) * stride, 0, 0) != 0);
}

// Bytes from row r0 to the end of the last valid row of a [rows, D] window
// of a tensor with row stride rs (elements), given N valid rows in total.
__device__ __forceinline__ int span_bytes(int r0, int rows, int N, int64_t rs, int D) {
  const int valid = min(rows, N - r0);
  return valid > 0 ? (int)(((int64_t)(valid - 1) * rs + D) * 2) : 0;
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

// blockIdx -> (sequence, head, query block) for packed variable-length
// batches, where the grid is sized by the longest sequence.  Query blocks go
// in descending order, each block index across all (sequence, head) pairs
// before the next: only long sequences own high block indices, so the
// heaviest work items start first (a non-causal block of a longer sequence
// also sees more keys), and every XCD draws the same mix of sequences.  Pair
// p stays on XCD p mod 8 when the pair count is a multiple of 8.
__device__ __forceinline__ WorkItem map_workgroup_packed(int wg, int nqb, int Hq, int pairs) {
  WorkItem w;
  w.qblk = nqb - 1 - wg / pairs;
  const int bh = wg % pairs;
  w.hq = bh % Hq;
  w.b = bh / Hq;
  return w;
}

}  // namespace eta
