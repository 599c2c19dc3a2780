// Shared device helpers of the attention kernels (forward, forward + JVP and
// backward): direct global -> LDS tile loads through buffer descriptors, the
// XOR slot swizzles of the two LDS tile layouts, and the 16x16x32 bf16 MFMA.
//
// Row tiles [64 tokens][dh] (K, V, Q or dO rows) put chunk c of row r in slot
// kslot(r, c); transposed tiles [dh][64 tokens] (V^T, K^T, Q^T, dO^T) put key
// chunk kc of row e in slot vslot(e, kc).  Both are involutions, so the same
// map turns an LDS slot back into the global chunk it holds.
#pragma once

#include "common.h"

namespace t2va {
namespace {

// 16-byte slot of chunk c of K row `row`.  The rows one 16-lane group reads
// together differ in bits 0, 1, 3, 4 (bit 2 is the sub-tile half); the XOR key
// spreads them over 16 bank groups.
template <int CPR>
__device__ __forceinline__ int kslot(int row, int c) {
  if constexpr (CPR == 16) return c ^ ((row & 3) | ((row >> 1) & 12));
  else return c ^ (((row >> 1) & 1) | ((row >> 2) & 6));   // 8 slots; row parity picks the half
}
// 16-byte slot of key chunk kc (8 keys) of V^T row e (64 keys = 8 chunks per row)
__device__ __forceinline__ int vslot(int e, int kc) { return kc ^ ((e >> 1) & 7); }

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over [base, base + bytes): loads past the end return zeros.
// Word 3 selects a 32-bit data format, as raw dword loads need on gfx9 parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from rsrc + voffset straight into LDS; lane i writes LDS
// bytes [dst + 16 i, dst + 16 i + 16) of a wave-uniform destination.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, bf16 *dst_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst_wave, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace
}  // namespace t2va
