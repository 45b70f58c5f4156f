// Score scan: every history key of every (sequence, KV head) dotted with the
// current query, max over the GQA group, written as fp32.
//
// What is computed: s[b][h][t] = max_g sum_j q[b][hG+g][j] K(b,h,t)[j]
// (ParisKV close-reading, section 一: s_i = <k_i, q>; the ECHO-OSDI26 wiki
// page's indexer scores all history keys before the exact top-k).
//
// gfx950 design.  The scan is HBM-bound: 256 B per bf16 key of d = 128.
//  * GQA groups (bf16, 2 <= G <= 16) use v_mfma_f32_16x16x32_bf16: the 16x32
//    A operand holds the G query rows (zero-padded), the 32x16 B operand holds
//    16 keys, four instructions cover d = 128.  A wave consumes one 16-token
//    block (4 KB) per step; each lane loads 4 x 16 B.  With G <= 4 the G scores
//    of a key land in one lane (C rows 0..3), so the group max needs no
//    cross-lane traffic.
//  * G = 1 and fp32 keys use the vector ALUs: 16 lanes share a key, each lane
//    owns one 16-byte piece, a wave loads 4 keys (1 KB contiguous in a pool
//    block) per instruction, and a 4-step DPP butterfly finishes each dot.
//  * Address resolution (block table / token table) happens per key inside
//    the scan; dead tokens are never read.
#include "skv_device.h"

namespace skv {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;  // tokens per workgroup (multiple of 16)

__device__ __forceinline__ u32x4_t ld16(const char* p) { return *(const u32x4_t*)p; }

// Score-key histogram of the tile (top 12 bits of the order-preserving key),
// built in LDS while scoring and added into the row's global histogram: the
// first digit of the exact top-k, fused into the scan.
struct HistArgs {
  const int32_t* lo;
  const int32_t* hi;
  uint32_t* hist;   // [B*H][4096]
};

__device__ __forceinline__ void hist_add(uint32_t* lh, float s, int t, int lo, int hi) {
  uint32_t u = __float_as_uint(s);
  if (t < lo || t >= hi || (u & 0x7f800000u) == 0x7f800000u) return;
  if (u == 0x80000000u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  atomicAdd(&lh[key >> 20], 1u);
}

__device__ __forceinline__ void hist_begin(uint32_t* lh) {
  for (int i = threadIdx.x; i < 4096; i += kThreads) lh[i] = 0u;
  __syncthreads();
}

__device__ __forceinline__ void hist_flush(uint32_t* lh, uint32_t* g) {
  __syncthreads();
  for (int i = threadIdx.x; i < 4096; i += kThreads) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(&g[i], c);
  }
}

template <bool BF16, int NPL, int GMAX, int U, bool HIST>
__global__ __launch_bounds__(kThreads) void score_valu_kernel(KvArgs kv, const void* qv, int G,
                                                               float* scores, HistArgs ha) {
  __shared__ uint32_t lh[HIST ? 4096 : 1];
  constexpr int E = BF16 ? 8 : 4;      // elements per 16-byte piece
  constexpr int ES = BF16 ? 2 : 4;     // bytes per element
  const int b = blockIdx.z, h = blockIdx.y;
  const int t_begin = blockIdx.x * kTile;
  const int t_end = min(kv.L_max, t_begin + kTile);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane & 15, sub = lane >> 4;
  const int NP = kv.d_k / E;           // pieces per row

  float qr[GMAX][NPL][E];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      const int pi = p + 16 * r;
      const bool on = g < G && pi < NP;
      const char* src = (const char*)qv +
                        ((((int64_t)b * kv.H + h) * G + (on ? g : 0)) * kv.d_k + pi * E) * ES;
      u32x4_t w = on ? ld16(src) : u32x4_t{0, 0, 0, 0};
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qr[g][r][2 * e] = bf16_lo(w[e]);
          qr[g][r][2 * e + 1] = bf16_hi(w[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qr[g][r][e] = __uint_as_float(w[e]);
      }
    }

  const char* kbase = (const char*)kv.k;
  float* srow = scores + ((int64_t)b * kv.H + h) * kv.L_max;
  const int n_groups = (t_end - t_begin + 3) >> 2;   // groups of 4 tokens
  int wlo = 0, whi = 0;
  if constexpr (HIST) {
    hist_begin(lh);
    wlo = ha.lo[b];
    whi = ha.hi[b];
  }

  for (int g0 = wave; g0 < n_groups; g0 += 4 * U) {
    u32x4_t kd[U][NPL];
    int tok[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t_begin + (g0 + 4 * u) * 4 + sub;
      tok[u] = t;
      const int64_t slot = (t < t_end) ? slot_of(kv, b, t) : -1;
      ok[u] = slot >= 0;
      const int64_t base = ok[u] ? row_elem(kv, b, h, slot, kv.d_k) : 0;
#pragma unroll
      for (int r = 0; r < NPL; ++r) {
        const int pi = p + 16 * r;
        kd[u][r] = (ok[u] && pi < NP) ? ld16(kbase + (base + pi * E) * ES) : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[GMAX];
#pragma unroll
      for (int g = 0; g < GMAX; ++g) acc[g] = 0.f;
#pragma unroll
      for (int r = 0; r < NPL; ++r) {
        float kf[E];
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[2 * e] = bf16_lo(kd[u][r][e]);
            kf[2 * e + 1] = bf16_hi(kd[u][r][e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) kf[e] = __uint_as_float(kd[u][r][e]);
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g] = fmaf(qr[g][r][e], kf[e], acc[g]);
      }
      float s = -INFINITY;
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        const float d = row16_sum(acc[g]);
        if (g < G) s = fmaxf(s, d);
      }
      if (p == 0 && tok[u] < t_end) {
        srow[tok[u]] = ok[u] ? s : -INFINITY;
        if constexpr (HIST) {
          if (ok[u]) hist_add(lh, s, tok[u], wlo, whi);
        }
      }
    }
  }
  if constexpr (HIST) hist_flush(lh, ha.hist + ((int64_t)b * kv.H + h) * 4096);
}

// bf16 keys, 2 <= G <= 16, d_k = 32 * NC.
template <int NC, int U, bool HIST>
__global__ __launch_bounds__(kThreads) void score_mfma_kernel(KvArgs kv, const uint16_t* q, int G,
                                                               float* scores, HistArgs ha) {
  __shared__ uint32_t lh[HIST ? 4096 : 1];
  const int b = blockIdx.z, h = blockIdx.y;
  const int t_begin = blockIdx.x * kTile;
  const int t_end = min(kv.L_max, t_begin + kTile);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int d_k = kv.d_k;

  // A operand: row m = n is query head n of the group (zero when n >= G);
  // lane group g4 of instruction j covers dims 8*(4j+g4) .. +8.
  bf16x8_t A[NC];
  const uint16_t* qrow = q + (((int64_t)b * kv.H + h) * G + (n < G ? n : 0)) * d_k;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    u32x4_t w = (n < G) ? ld16((const char*)(qrow + (4 * j + g4) * 8)) : u32x4_t{0, 0, 0, 0};
    A[j] = __builtin_bit_cast(bf16x8_t, w);
  }

  const char* kbase = (const char*)kv.k;
  float* srow = scores + ((int64_t)b * kv.H + h) * kv.L_max;
  const int n_chunks = (t_end - t_begin + 15) >> 4;
  int wlo = 0, whi = 0;
  if constexpr (HIST) {
    hist_begin(lh);
    wlo = ha.lo[b];
    whi = ha.hi[b];
  }

  for (int c0 = wave; c0 < n_chunks; c0 += 4 * U) {
    bf16x8_t Bm[U][NC];
    int tok[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      const int t = t_begin + c * 16 + n;
      tok[u] = (c < n_chunks) ? t : t_end;
      const int64_t slot = (c < n_chunks && t < t_end) ? slot_of(kv, b, t) : -1;
      ok[u] = slot >= 0;
      const int64_t base = ok[u] ? row_elem(kv, b, h, slot, d_k) : 0;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        u32x4_t w = ok[u] ? ld16(kbase + (base + (4 * j + g4) * 8) * 2) : u32x4_t{0, 0, 0, 0};
        Bm[u][j] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NC; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[j], Bm[u][j], acc, 0, 0, 0);
      // lane (n, g4) holds C[4*g4 + i][n]: query head 4*g4+i against key n
      float s = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g4 + i < G) s = fmaxf(s, acc[i]);
      if (G > 4) {
        s = fmaxf(s, __shfl_xor(s, 16, 64));
        s = fmaxf(s, __shfl_xor(s, 32, 64));
      }
      if (g4 == 0 && tok[u] < t_end) {
        srow[tok[u]] = ok[u] ? s : -INFINITY;
        if constexpr (HIST) {
          if (ok[u]) hist_add(lh, s, tok[u], wlo, whi);
        }
      }
    }
  }
  if constexpr (HIST) hist_flush(lh, ha.hist + ((int64_t)b * kv.H + h) * 4096);
}

template <bool BF16, int NPL, int GMAX, int U>
void launch_valu_k(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                   dim3 grid, hipStream_t s) {
  if (ha.hist)
    score_valu_kernel<BF16, NPL, GMAX, U, true><<<grid, kThreads, 0, s>>>(kv, q, G, scores, ha);
  else
    score_valu_kernel<BF16, NPL, GMAX, U, false><<<grid, kThreads, 0, s>>>(kv, q, G, scores, ha);
}

template <bool BF16, int NPL, int GCAP>
hipError_t launch_valu(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                       dim3 grid, hipStream_t s) {
  if (G == 1)
    launch_valu_k<BF16, NPL, 1, 4>(kv, q, G, scores, ha, grid, s);
  else if (GCAP >= 2 && G == 2)
    launch_valu_k<BF16, NPL, (GCAP >= 2 ? 2 : 1), 4>(kv, q, G, scores, ha, grid, s);
  else if (GCAP >= 4 && G <= 4)
    launch_valu_k<BF16, NPL, (GCAP >= 4 ? 4 : 1), 2>(kv, q, G, scores, ha, grid, s);
  else if (GCAP >= 8 && G <= 8)
    launch_valu_k<BF16, NPL, (GCAP >= 8 ? 8 : 1), 2>(kv, q, G, scores, ha, grid, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int NC, int U>
void launch_mfma_k(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                   dim3 grid, hipStream_t s) {
  if (ha.hist)
    score_mfma_kernel<NC, U, true><<<grid, kThreads, 0, s>>>(kv, (const uint16_t*)q, G, scores, ha);
  else
    score_mfma_kernel<NC, U, false><<<grid, kThreads, 0, s>>>(kv, (const uint16_t*)q, G, scores, ha);
}

}  // namespace

hipError_t launch_score(const KvArgs& kv, const void* q, int G, float* scores, const int32_t* lo,
                        const int32_t* hi, uint32_t* hist, hipStream_t s) {
  dim3 grid((kv.L_max + kTile - 1) / kTile, kv.H, kv.B);
  HistArgs ha{lo, hi, hist};
  if (kv.bf16 && G >= 2 && G <= 16 && kv.d_k % 32 == 0) {
    switch (kv.d_k / 32) {
      case 2: launch_mfma_k<2, 2>(kv, q, G, scores, ha, grid, s); break;
      case 4: launch_mfma_k<4, 2>(kv, q, G, scores, ha, grid, s); break;
      case 8: launch_mfma_k<8, 2>(kv, q, G, scores, ha, grid, s); break;
      case 18: launch_mfma_k<18, 1>(kv, q, G, scores, ha, grid, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int E = kv.bf16 ? 8 : 4;
  const int npl = (kv.d_k / E + 15) / 16;
  if (kv.bf16) {
    if (npl == 1) return launch_valu<true, 1, 8>(kv, q, G, scores, ha, grid, s);
    if (npl == 2) return launch_valu<true, 2, 4>(kv, q, G, scores, ha, grid, s);
    if (npl <= 5) return launch_valu<true, 5, 1>(kv, q, G, scores, ha, grid, s);
  } else {
    if (npl == 1) return launch_valu<false, 1, 8>(kv, q, G, scores, ha, grid, s);
    if (npl == 2) return launch_valu<false, 2, 8>(kv, q, G, scores, ha, grid, s);
    if (npl <= 4) return launch_valu<false, 4, 2>(kv, q, G, scores, ha, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skv
