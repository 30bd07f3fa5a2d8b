// LDS tile layouts and fragment reads shared by the prefill attention kernels (gfx950, wave64):
// the selected-chunk attention (attention.hip) and the dense causal comparator (dense.hip) stage
// one 64-key chunk of K and V at a time in these layouts.
#pragma once
#include "hils_device.h"

namespace hils {

// LDS layout of one stage.  K: row-major, rows padded by 16 bytes so the 16 rows of an MFMA
// operand read fall on distinct banks.  V: d-block-major [d/16][row][16 elements], each d-block
// padded by 32 bytes, so a transpose read (8 rows x 32 bytes) and the staging writes are
// conflict-free.
template <typename T, int D>
struct AttnLayout {
  static constexpr int RB = D * (int)sizeof(T);       // row bytes
  static constexpr int VPR = RB / 16;                 // 16-byte vectors per row
  static constexpr int KLD = RB + 16;                 // K row stride (bytes)
  static constexpr int VDB = 64 * 16 * (int)sizeof(T) + 32;   // V d-block stride (bytes)
  static constexpr int KBYTES = 64 * KLD;
  static constexpr int VBYTES = (D / 16) * VDB;
};

// K tile of the bf16 one-block kernels.  At d = 128: 256-byte rows whose 16-byte vectors are
// XOR-permuted by the row, so that a 16x16x32 A-fragment read (lane (m, g): row 16 kb + m,
// vector 4 g + st) touches every LDS bank once; rows padded by 16 bytes instead conflict two
// ways on gfx950 (measured: 127 against 243 bytes per clock per CU).  Other d keep padded rows.
template <int D>
struct BlockKLayout {
  static constexpr int RB = D * 2;
  static constexpr bool kSwz = D == 128;
  static constexpr int LD = kSwz ? RB : RB + 16;
  __device__ static __forceinline__ int off(int row, int vec) {
    if constexpr (kSwz) return row * RB + ((vec ^ (((row & 3) << 2) | ((row >> 2) & 3))) << 4);
    else return row * LD + vec * 16;
  }
};
static_assert(64 * BlockKLayout<128>::LD <= AttnLayout<bf16, 128>::KBYTES, "K tile fits its stage");

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// PV A-operand fragment (bf16) for d-block db and step st.  Slot z of lane group g holds key
// 16*(i/4) + 4g + i%4 with i = 8*st + z (the S^T output layout).  Transpose read: lane L of each
// 16-lane group supplies 4 elements of row (base + L/4) at column 4*(L%4) of the d-block, and
// lane i of the group receives column i of those four rows.
template <int VDB>
__device__ __forceinline__ bf16x8 v_frag_bf16(const char* vbuf, int lane16, int g, int db, int st) {
  const char* p0 = vbuf + db * VDB + (32 * st + 4 * g + (lane16 >> 2)) * 32 + 8 * (lane16 & 3);
  const char* p1 = p0 + 16 * 32;
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const void*)p0);
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const void*)p1);
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// fp32: one element per step, key 16*(st/4) + 4g + st%4, column 16*db + lane16.
template <int VDB>
__device__ __forceinline__ float v_frag_f32(const char* vbuf, int lane16, int g, int db, int st) {
  const int row = 16 * (st >> 2) + 4 * g + (st & 3);
  return *reinterpret_cast<const float*>(vbuf + db * VDB + row * 64 + lane16 * 4);
}

// First key (or value) row of chunk j: `base` + j * 64 rows for contiguous [.., L, d] rows of
// one key/value head, or page bt[j] (clamped to the pool) of a pool [pages, Hk, 64, d] at
// `pool` for key/value head kvh.
template <typename T, int D>
__device__ __forceinline__ const T* kv_chunk(const T* base, const T* pool, const int32_t* bt, int num_pages, int Hk,
                                             int kvh, int j) {
  if (bt == nullptr) return base + (size_t)j * 64 * D;
  const int pg = min(max(bt[j], 0), num_pages - 1);
  return pool + ((size_t)pg * Hk + kvh) * 64 * D;
}

}  // namespace hils
