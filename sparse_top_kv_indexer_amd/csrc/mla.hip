// Shared-latent (MLA-style) sparse attention on matrix cores.
//
// What is computed (v == NULL in skv_kv): every query head g of KV head h
// attends over the same latent rows; the logit is scale * q_g . latent_t over
// all d_k = 576 dims and the value is the first d_v = 512 dims of the latent
// row.  A = selected ∪ sink ∪ local exactly as in sparsekv_gather_attend.
// (ECHO-OSDI26 wiki page, problem and motivation: DSA keeps an MLA latent KV
// plus a separate indexer K cache; the indexer picks the top-k tokens and
// attention runs over those tokens only.)
//
// gfx950 design.  With 128 query heads sharing one latent row the step is a
// real dense contraction: 2 x 128 x 576 x k flops for the logits and the same
// order for P.V, on 1152-byte rows.  A workgroup (G/16 waves, 16 heads per
// wave) owns one split of the position list: it stages up to 64 latent rows
// in LDS once, then per 16-token chunk
//   S^T[16 tokens x 16 heads] = K_chunk . Q^T     18 x v_mfma_f32_16x16x32_bf16
// so each lane ends up with P[head][4 tokens] in exactly the A-operand layout
// of the value product, and
//   O[16 heads x 512] += P . V                    32 x v_mfma_f32_16x16x16_bf16
// with P split into a bf16 head and a bf16 tail (two products), which keeps
// the probabilities to ~16 significant bits.  The value operand is read from
// a transposed copy of the chunk in LDS.  An online softmax (log2 domain)
// runs across chunks; the split partials are merged exactly by log-sum-exp.
#include <algorithm>

#include "skv_device.h"

namespace skv {

namespace {

constexpr int kDk = 576, kDv = 512;
constexpr int kRowPad = kDk + 8;        // LDS row stride (bf16 elements)
constexpr int kStage = 64;              // latent rows staged per LDS fill
constexpr int kNC = kDk / 32;           // 18 MFMA k-steps for the logits
constexpr int kVB = kDv / 16;           // 32 value column blocks

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mla_split_kernel(
    KvArgs kv, const uint16_t* q, int G, const int32_t* idx, int k, const int32_t* lo_p,
    const int32_t* hi_p, float scale_log2, int n_split, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t rows[kStage * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kDv * 16];    // [dim][token]
  __shared__ int64_t roff[kStage];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int head0 = wave * 16;                    // this wave's first query head

  // Q^T operand: lane (n, g4), step j holds q[head0 + n][8 (4j + g4) .. +8]
  bf16x8_t Qf[kNC];
  const uint16_t* qrow = q + (((int64_t)b * kv.H + h) * G + head0 + n) * kDk;
#pragma unroll
  for (int j = 0; j < kNC; ++j)
    Qf[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qrow + 8 * (4 * j + g4)));

  const int seq = min(kv.seq_len[b], kv.L_max);
  const int lo = max(0, min(lo_p[b], seq));
  const int hi = max(lo, min(hi_p[b], seq));
  const int n_list = k + lo + (seq - hi);
  const int chunk = (n_list + n_split - 1) / n_split;
  const int p0 = s * chunk, p1 = min(n_list, p0 + chunk);
  const int32_t* irow = idx + ((int64_t)b * kv.H + h) * k;

  // online softmax state for head head0 + n (replicated over g4)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t O[kVB];
#pragma unroll
  for (int c = 0; c < kVB; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kb = (const uint16_t*)kv.k;
  for (int q0 = p0; q0 < p1; q0 += kStage) {
    const int cnt = min(kStage, p1 - q0);
    if (tid < kStage) {
      int64_t ro = -1;
      if (tid < cnt) {
        const int pos = q0 + tid;
        int t;
        if (pos < k) {
          t = irow[pos];
          if (t < lo || t >= hi) t = -1;
        } else if (pos - k < lo) {
          t = pos - k;
        } else {
          t = hi + (pos - k - lo);
        }
        const int64_t slot = t >= 0 ? slot_of(kv, b, t) : -1;
        ro = slot >= 0 ? row_elem(kv, b, h, slot, kDk) : -1;
      }
      roff[tid] = ro;
    }
    __syncthreads();
    // stage the rows: 72 pieces of 16 B per row.  With up to four waves each
    // thread keeps four loads in flight before their LDS stores; eight waves
    // have no registers to spare and issue one load per store.
    {
      constexpr int kPieces = kStage * (kDk / 8);
      if constexpr (WAVES >= 8) {
        for (int i = tid; i < kPieces; i += WAVES * 64) {
          const int r = i / (kDk / 8), pc = i - r * (kDk / 8);
          const int64_t ro = roff[r];
          const u32x4_t v = ro >= 0 ? *(const u32x4_t*)(kb + ro + 8 * pc) : u32x4_t{0, 0, 0, 0};
          *(u32x4_t*)(rows + r * kRowPad + 8 * pc) = v;
        }
      } else {
        constexpr int kB = 4;
        for (int i0 = 0; i0 < kPieces; i0 += kB * WAVES * 64) {
          u32x4_t v[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u) {
            const int i = i0 + u * WAVES * 64 + tid;
            const int r = i / (kDk / 8), pc = i - r * (kDk / 8);
            const int64_t ro = i < kPieces ? roff[r] : -1;
            v[u] = ro >= 0 ? *(const u32x4_t*)(kb + ro + 8 * pc) : u32x4_t{0, 0, 0, 0};
          }
#pragma unroll
          for (int u = 0; u < kB; ++u) {
            const int i = i0 + u * WAVES * 64 + tid;
            const int r = i / (kDk / 8), pc = i - r * (kDk / 8);
            if (i < kPieces) *(u32x4_t*)(rows + r * kRowPad + 8 * pc) = v[u];
          }
        }
      }
    }
    __syncthreads();

    for (int c0 = 0; c0 < cnt; c0 += 16) {
      // transposed value copy of this chunk: vt[dim][token]
      for (int d = tid; d < kDv; d += WAVES * 64) {
        uint32_t pk[8];
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2)
          pk[t2] = (uint32_t)rows[(c0 + 2 * t2) * kRowPad + d] |
                   ((uint32_t)rows[(c0 + 2 * t2 + 1) * kRowPad + d] << 16);
        *(u32x4_t*)(vt + d * 16) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
        *(u32x4_t*)(vt + d * 16 + 8) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
      }
      __syncthreads();
      // S^T[token 4 g4 + i][head n] for the 16 tokens of the chunk
      f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kNC; ++j) {
        const bf16x8_t Kf = __builtin_bit_cast(
            bf16x8_t, *(const u32x4_t*)(rows + (c0 + n) * kRowPad + 8 * (4 * j + g4)));
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf, Qf[j], S, 0, 0, 0);
      }
      float z[4];
      float cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = c0 + 4 * g4 + i;
        const bool ok = tk < cnt && roff[tk] >= 0;
        z[i] = ok ? S[i] * scale_log2 : -INFINITY;
        cm = fmaxf(cm, z[i]);
      }
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float m_new = fmaxf(m_run, cm);
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = m_new == -INFINITY ? 0.f : exp2f(z[i] - m_new);
        ps += p[i];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      const float corr = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run = l_run * corr + ps;
      m_run = m_new;
      // O rows are heads 4 g4 + i: fetch their correction factors
      float oc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) oc[i] = __shfl(corr, 4 * g4 + i, 64);
      // P as the A operand (head n, tokens 4 g4 .. +3), split into head + tail
      uint32_t hi16[4], lo16[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi16[i] = f32_to_bf16_rne(p[i]);
        lo16[i] = f32_to_bf16_rne(p[i] - __uint_as_float(hi16[i] << 16));
      }
      const bf16x4_t Ph = __builtin_bit_cast(
          bf16x4_t, u32x2_t{hi16[0] | (hi16[1] << 16), hi16[2] | (hi16[3] << 16)});
      const bf16x4_t Pl = __builtin_bit_cast(
          bf16x4_t, u32x2_t{lo16[0] | (lo16[1] << 16), lo16[2] | (lo16[3] << 16)});
#pragma unroll
      for (int c = 0; c < kVB; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[c][i] *= oc[i];
        const bf16x4_t Vf = __builtin_bit_cast(
            bf16x4_t, *(const u32x2_t*)(vt + (16 * c + n) * 16 + 4 * g4));
        O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ph, Vf, O[c], 0, 0, 0);
        O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Pl, Vf, O[c], 0, 0, 0);
      }
      __syncthreads();
    }
    __syncthreads();
  }

  // partial of this split: O[head][512], max, sum (lane holds rows 4 g4 + i)
  const int stride = kDv + 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = head0 + 4 * g4 + i;
    float* dst = part + ((((int64_t)b * kv.H + h) * G + hd) * n_split + s) * stride;
#pragma unroll
    for (int c = 0; c < kVB; ++c) dst[16 * c + n] = O[c][i];
  }
  if (g4 == 0) {
    float* dst = part + ((((int64_t)b * kv.H + h) * G + head0 + n) * n_split + s) * stride;
    dst[kDv] = m_run;
    dst[kDv + 1] = l_run;
  }
}

int mla_splits(int k) { return std::max(1, std::min(64, (k + kStage - 1) / kStage)); }

}  // namespace

bool mla_supported(const KvArgs& kv, int G) {
  return kv.bf16 && kv.v == nullptr && kv.d_k == kDk && kv.d_v == kDv &&
         (G == 16 || G == 32 || G == 64 || G == 128);
}

size_t mla_workspace_bytes(const KvArgs& kv, int G, int k) {
  return (size_t)kv.B * kv.H * G * mla_splits(k) * (kDv + 2) * sizeof(float);
}

hipError_t launch_mla_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                             const int32_t* lo, const int32_t* hi, float scale, float* out,
                             void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  const int n_split = mla_splits(k);
  float* part = (float*)ws;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(n_split, kv.H, kv.B);
  const uint16_t* qq = (const uint16_t*)q;
  switch (G / 16) {
    case 1: mla_split_kernel<1><<<grid, 64, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part); break;
    case 2: mla_split_kernel<2><<<grid, 128, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part); break;
    case 4: mla_split_kernel<4><<<grid, 256, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part); break;
    case 8: mla_split_kernel<8><<<grid, 512, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_reduce(part, n_split, kDv, kv.H * G, kv.B, out, st);
}

}  // namespace skv
