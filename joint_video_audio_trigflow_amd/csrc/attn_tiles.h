// Shared helpers of the attention kernels (forward, forward + JVP and
// backward): direct global -> LDS tile loads through buffer descriptors, the
// XOR slot swizzles of the two LDS tile layouts, the 16x16x32 bf16 MFMA, and
// the tail split of a launch (work decomposition and its host-side plan).
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

// ---------------------------------------------------------------------------
// Tail split.  These kernels run one workgroup per compute unit at a time, so
// each XCD runs its tiles in rounds, and a last round with few tiles leaves
// most of the XCD idle.  Each XCD therefore runs its first n_full tiles whole
// and cuts its last `rem` tiles into k pieces over consecutive ranges of
// stages (64 or 128 tokens) of the streamed operand, dispatched after every
// whole tile.
// Each piece stores a partial result into scratch and a second kernel merges
// the pieces of every split tile in piece order.
// ---------------------------------------------------------------------------
// The forward kernels cut a tile into at most 8 pieces; the backward kernels,
// whose pieces each store fp32 partials of a whole tile (dK and dV: 1 KB per
// key row), at most 4 (8 was 1.7 % slower for the standard workload's
// backward, 0.6 % faster at high-res).
constexpr int kMaxPieces = 8;
constexpr int kMaxPiecesBwd = 4;
constexpr int kMinPieceKeys = 512;   // no piece shorter than 512 keys (at the longest sample)
constexpr int kMaxDevices = 64;
struct SplitArgs {
  int n_full, rem, k;
  int pbank;   // forward with a prefix output: pieces before the second (prefix) bank
};

// Workgroup w of a split launch: hardware places w on XCD w % 8, and each XCD
// gets a contiguous range of per_xcd logical tiles (so one head's streamed
// operands stay in that XCD's L2).  Its first n_full workgroups run tiles
// whole; the next rem * k run the remaining tiles as k pieces each.  slot is
// the split tile's index among all split tiles (-1: a whole tile).
struct SplitItem {
  int L, piece, slot;
};
__host__ __device__ __forceinline__ SplitItem split_item(int w, int per_xcd, const SplitArgs &sp) {
  const int xcd = w & 7, wi = w >> 3;
  if (wi < sp.n_full) return {xcd * per_xcd + wi, 0, -1};
  const int tt = (wi - sp.n_full) / sp.k;
  return {xcd * per_xcd + sp.n_full + tt, wi - sp.n_full - tt * sp.k, xcd * sp.rem + tt};
}
// the logical tile of split slot `slot` (merge kernels: one workgroup per slot)
__host__ __device__ __forceinline__ int split_tile(int slot, int per_xcd, const SplitArgs &sp) {
  const int xcd = slot / sp.rem;
  return xcd * per_xcd + sp.n_full + (slot - xcd * sp.rem);
}
// stages [s0, s1) of piece `piece` of k over nst stages (empty when nst < k)
__host__ __device__ __forceinline__ void piece_stages(int nst, int piece, int k, int &s0, int &s1) {
  s0 = piece * nst / k;
  s1 = (piece + 1) * nst / k;
}

// The split of an XCD's per_xcd tiles when it holds `slots` workgroups at
// once: the k <= max_k (<= kMaxPieces) that minimises the time of the last round(s),
// ceil(rem k / slots) / k whole-tile times, ties to the smaller k; no split
// when nothing is gained, a piece would span fewer than min_stages of the
// nst_max stages, or the scratch holds fewer than 8 rem k pieces.
inline SplitArgs plan_split(int per_xcd, int slots, int nst_max, size_t cap_pieces, int min_stages,
                            int max_k = kMaxPieces) {
  SplitArgs sp{per_xcd, 0, 1, 0};
  if (slots <= 0) return sp;
  const int rem = per_xcd % slots;
  if (rem == 0) return sp;
  int best_k = 1;
  int64_t best_num = 1, best_den = 1;   // cost as the fraction ceil(rem k / slots) / k
  for (int k = 2; k <= max_k && k <= kMaxPieces; ++k) {
    if (nst_max / k < min_stages || (size_t)8 * rem * k > cap_pieces) break;
    const int64_t num = (rem * k + slots - 1) / slots;
    if (num * best_den < best_num * k) {
      best_k = k;
      best_num = num;
      best_den = k;
    }
  }
  if (best_k == 1) return sp;
  sp.n_full = per_xcd - rem;
  sp.rem = rem;
  sp.k = best_k;
  return sp;
}

// Workgroups of `kernel` (threads, dynamic LDS) one XCD holds at once, 0 if
// unknown; queried once per device into `cache` (0: not yet, -1: unknown).
template <typename Kernel>
int xcd_slots(Kernel kernel, int threads, size_t lds, int (&cache)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    const bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) == hipSuccess;
    if (!ok) (void)hipGetLastError();
    cache[dev] = (ok && cus >= 8 && per_cu >= 1) ? per_cu * (cus / 8) : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

}  // namespace
}  // namespace t2va
