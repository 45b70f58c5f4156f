// Device-side helpers shared by the gfx950 kernels of the sparse decode step:
// KV addressing (block table / token table / contiguous), bf16 unpacking and
// 16-lane DPP reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skv_internal.h"

namespace skv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Physical slot of logical token t of sequence b, or -1 when the token is dead
// or t >= seq_len[b].  Paged: block_table[b][t/16]*16 + t%16 (16-token
// blocks); token table: token_table[b][t] (vToken reading notes, Eq. (2));
// contiguous: t itself.
__device__ __forceinline__ int64_t slot_of(const KvArgs& kv, int b, int t) {
  if (t < 0 || t >= kv.seq_len[b] || t >= kv.L_max) return -1;
  if (kv.token_table) return (int64_t)kv.token_table[(int64_t)b * kv.L_max + t];
  if (kv.block_table)
    return (int64_t)kv.block_table[(int64_t)b * (kv.L_max >> 4) + (t >> 4)] * 16 + (t & 15);
  return t;
}

// Element offset of the row (slot, head h) in a store whose rows have `d`
// elements: pools are [n_blocks][H][16][d], contiguous stores [B][H][L_max][d].
__device__ __forceinline__ int64_t row_elem(const KvArgs& kv, int b, int h, int64_t slot, int d) {
  if (kv.block) return (((slot >> 4) * kv.H + h) * 16 + (slot & 15)) * (int64_t)d;
  return (((int64_t)b * kv.H + h) * kv.L_max + slot) * (int64_t)d;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row.  The partner of each step is a lane
// permutation that is its own inverse (xor 15, xor 7, xor 2, xor 1 within the
// row), so both partners add the same two operands and every lane ends with
// bit-identical totals.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0x140>(x);   // row_mirror        (lane ^ 15)
  x += dpp_f<0x141>(x);   // row_half_mirror   (lane ^ 7)
  x += dpp_f<0x4E>(x);    // quad_perm 2,3,0,1 (lane ^ 2)
  x += dpp_f<0xB1>(x);    // quad_perm 1,0,3,2 (lane ^ 1)
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0x140>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0xB1>(x));
  return x;
}

__device__ __forceinline__ int wave_lane() { return (int)__lane_id(); }

// Exclusive prefix sum over a 64-lane wave (every lane holds one value).
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

// One 16-byte global load.
__device__ __forceinline__ u32x4_t ld16(const char* p) { return *(const u32x4_t*)p; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele
// shifts of 1, 2, 4, 8 inside each 16-lane row (lanes without a source add
// 0), then lane 15 of each row into the next row and lane 31 into rows 2, 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations and meets the other waves, without waiting for its
// outstanding global loads, stores or atomics (__syncthreads() waits for
// those as well).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy n 4-byte words from global memory to LDS with up to PER loads per
// thread in flight at once (a plain copy loop waits for every load before its
// LDS store, one memory latency per iteration).
template <int PER>
__device__ __forceinline__ void stage_words(uint32_t* dst, const uint32_t* src, int n, int tid,
                                            int nthreads) {
  for (int base = 0; base < n; base += PER * nthreads) {
    uint32_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + u * nthreads + tid;
      v[u] = i < n ? src[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + u * nthreads + tid;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id (XCD =
// id % 8), and each XCD has its own L2.  For n (a multiple of 8) workgroups,
// xcd_remap(id, n) gives the virtual index under which XCD x runs the
// consecutive virtual indices [x n / 8, (x + 1) n / 8), so workgroups that
// read the same data can be placed on one XCD.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int id, int n) {
  return (id % kXcds) * (n / kXcds) + id / kXcds;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace skv
