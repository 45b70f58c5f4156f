// Gather + split-k sparse attention and the exact split merge.
//
// What is computed, for each sequence b, KV head h and query head g:
//   A   = {idx[b][h][i] in [lo, hi), live} ∪ {live t < lo} ∪ {live t >= hi}
//   out = sum_{t in A} softmax_t(scale q.K_t) V_t
// ParisKV close-reading, section 一 (paper Eqs. (1)-(3)): softmax is
// recomputed over the full-precision KV of the selected set; section 2.5:
// sink and local regions are attended densely next to the retrieved set.
// Rows are reached through the slot mapping (vToken reading notes, section
// 3.4, Eq. (2)).
//
// gfx950 design.  The positions of A form a virtual list
// [idx[0..k) | 0..lo-1 | hi..seq_len-1] that is cut into n_split contiguous
// splits; a 256-thread workgroup owns one (b, h, split).  Inside it, sixteen
// 16-lane rows each stream their own tokens (16 B of K and 16 B of V per lane
// for d = 128 bf16), finish the G dot products with a DPP butterfly and keep a
// running (max, sum, weighted values) per query head in the log2 domain.  The
// rows and waves are merged by log-sum-exp at the end and written as one
// partial per split; attend_reduce_kernel merges the splits exactly.
#include "skv_device.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = kThreads / 16;   // 16-lane rows per workgroup


template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4_t w, float* f) {
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(w[e]);
      f[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  }
}

// Merge (m2, l2, a2) into (m1, l1, a1); log2-domain maxima, -inf = empty.
__device__ __forceinline__ void lse_merge(float& m1, float& l1, float* a1, float m2, float l2,
                                          const float* a2, int n) {
  const float m = fmaxf(m1, m2);
  if (m == -INFINITY) return;
  const float c1 = exp2f(m1 - m), c2 = exp2f(m2 - m);
  l1 = l1 * c1 + l2 * c2;
  for (int i = 0; i < n; ++i) a1[i] = a1[i] * c1 + a2[i] * c2;
  m1 = m;
}

// With out != nullptr (n_split == 1) the workgroup writes the normalised
// output itself, out = acc / l (0 for an empty row) -- what the merge would
// compute from its one partial -- and no merge kernel follows.
template <bool BF16, int NPL, int GMAX>
__global__ __launch_bounds__(kThreads) void attend_split_kernel(
    KvArgs kv, const void* qv, int G, const int32_t* idx, int k, const int32_t* lo_p,
    const int32_t* hi_p, float scale_log2, int n_split, float* part, float* out) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int PE = NPL * E;            // elements of a row held by one lane
  constexpr int NB = NPL == 1 ? 8 : 4;   // tokens whose loads are in flight per row
  __shared__ int64_t rows_sh[kThreads];  // element offsets of this piece's rows (-1 = skip)
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane & 15;
  const int row = wave * 4 + (lane >> 4);
  const int D = kv.d_k;

  float qr[GMAX][PE];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      const bool on = g < G;
      const char* src = (const char*)qv +
          ((((int64_t)b * kv.H + h) * G + (on ? g : 0)) * D + (p + 16 * r) * E) * ES;
      u32x4_t w = on ? ld16(src) : u32x4_t{0, 0, 0, 0};
      unpack<BF16>(w, &qr[g][r * E]);
    }

  const int seq = min(kv.seq_len[b], kv.L_max);
  const int lo = max(0, min(lo_p[b], seq));
  const int hi = max(lo, min(hi_p[b], seq));
  const int n_list = k + lo + (seq - hi);
  const int chunk = (n_list + n_split - 1) / n_split;
  const int p0 = s * chunk, p1 = min(n_list, p0 + chunk);
  const int32_t* irow = idx + ((int64_t)b * kv.H + h) * k;

  float m[GMAX], l[GMAX], acc[GMAX][PE];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < PE; ++e) acc[g][e] = 0.f;
  }

  const char* kb = (const char*)kv.k;
  const char* vb = (const char*)kv.v;
  for (int q0 = p0; q0 < p1; q0 += kThreads) {
    const int cnt = min(kThreads, p1 - q0);
    // resolve this piece's positions to row offsets, one position per thread
    if ((int)threadIdx.x < cnt) {
      const int pos = q0 + threadIdx.x;
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
      rows_sh[threadIdx.x] = slot >= 0 ? row_elem(kv, b, h, slot, D) : -1;
    }
    __syncthreads();
    for (int j0 = row; j0 < cnt; j0 += kRows * NB) {
      u32x4_t kd[NB][NPL], vd[NB][NPL];
      int64_t ro[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int j = j0 + u * kRows;
        ro[u] = j < cnt ? rows_sh[j] : -1;
#pragma unroll
        for (int r = 0; r < NPL; ++r) {
          if (ro[u] >= 0) {
            kd[u][r] = ld16(kb + (ro[u] + (p + 16 * r) * E) * ES);
            vd[u][r] = ld16(vb + (ro[u] + (p + 16 * r) * E) * ES);
          } else {
            kd[u][r] = u32x4_t{0, 0, 0, 0};
            vd[u][r] = u32x4_t{0, 0, 0, 0};
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (ro[u] < 0) continue;            // uniform within the 16-lane row
        float kf[PE], vf[PE];
#pragma unroll
        for (int r = 0; r < NPL; ++r) {
          unpack<BF16>(kd[u][r], &kf[r * E]);
          unpack<BF16>(vd[u][r], &vf[r * E]);
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
          if (g >= G) break;
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < PE; ++e) d = fmaf(qr[g][e], kf[e], d);
          const float z = row16_sum(d) * scale_log2;
          const float mn = fmaxf(m[g], z);
          const float corr = exp2f(m[g] - mn);   // 0 when m was -inf
          const float pz = exp2f(z - mn);
          l[g] = l[g] * corr + pz;
#pragma unroll
          for (int e = 0; e < PE; ++e) acc[g][e] = fmaf(pz, vf[e], acc[g][e] * corr);
          m[g] = mn;
        }
      }
    }
    __syncthreads();
  }

  // merge the four rows of each wave (lanes p, p+16, p+32, p+48)
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float m2 = __shfl_xor(m[g], x, 64);
      const float l2 = __shfl_xor(l[g], x, 64);
      float a2[PE];
#pragma unroll
      for (int e = 0; e < PE; ++e) a2[e] = __shfl_xor(acc[g][e], x, 64);
      lse_merge(m[g], l[g], acc[g], m2, l2, a2, PE);
    }
  }

  // merge the four waves through LDS: [wave][g][D + 2]
  extern __shared__ float red[];
  const int stride = D + 2;
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      float* dst = red + ((size_t)wave * G + g) * stride;
#pragma unroll
      for (int r = 0; r < NPL; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) dst[(p + 16 * r) * E + e] = acc[g][r * E + e];
      if (p == 0) {
        dst[D] = m[g];
        dst[D + 1] = l[g];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, j = i - g * D;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[((size_t)w * G + g) * stride + D]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float* src = red + ((size_t)w * G + g) * stride;
        const float c = exp2f(src[D] - mm);
        ll += src[D + 1] * c;
        aa += src[j] * c;
      }
    }
    if (out) {
      const float inv_l = ll > 0.f ? 1.f / ll : 0.f;
      out[(((int64_t)b * kv.H + h) * G + g) * D + j] = aa * inv_l;
      continue;
    }
    float* dst = part + ((((int64_t)b * kv.H + h) * G + g) * n_split + s) * stride;
    dst[j] = aa;
    if (j == 0) {
      dst[D] = mm;
      dst[D + 1] = ll;
    }
  }
}

// bf16, d_k = d_v = 128, 1 <= G <= GMAX <= 16.  A wave takes 16 attended
// tokens at a time: the logits come from matrix cores as
//   S^T[16 tokens x 16 heads] = K_chunk . Q^T   (4 x v_mfma_f32_16x16x32_bf16)
// so lane (n, g4) holds the four logits of query head n for tokens 4 g4 .. +3,
// the softmax statistics need only a max / sum over the lane and its three
// partners, and the value product runs on the vector ALUs with every lane
// owning two output dims of every head: per token one 256-byte value row is
// read by the whole wave (4 B per lane) and each probability is broadcast from
// the lane that holds it (v_readlane).  Two chunks' rows are in flight per
// wave.
template <int GMAX>
__global__ __launch_bounds__(kThreads) void attend_mfma_kernel(
    KvArgs kv, const uint16_t* q, int G, const int32_t* idx, int k, const int32_t* lo_p,
    const int32_t* hi_p, float scale_log2, int n_split, float* part) {
  constexpr int D = 128;
  constexpr int CH = 2;                  // chunks of 16 tokens in flight per wave
  __shared__ int64_t rows_sh[kThreads];
  __shared__ float red[4][GMAX][D + 2];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g4 = lane >> 4;

  bf16x8_t Qf[4];
  {
    const uint16_t* qrow = q + (((int64_t)b * kv.H + h) * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t w = n < G ? ld16((const char*)(qrow + 8 * (4 * j + g4))) : u32x4_t{0, 0, 0, 0};
      Qf[j] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int seq = min(kv.seq_len[b], kv.L_max);
  const int lo = max(0, min(lo_p[b], seq));
  const int hi = max(lo, min(hi_p[b], seq));
  const int n_list = k + lo + (seq - hi);
  const int chunk = (n_list + n_split - 1) / n_split;
  const int p0 = s * chunk, p1 = min(n_list, p0 + chunk);
  const int32_t* irow = idx + ((int64_t)b * kv.H + h) * k;

  float m_run = -INFINITY, l_run = 0.f;     // head n (lanes n < G)
  float acc[GMAX][2];                       // dims 2 lane, 2 lane + 1 of every head
#pragma unroll
  for (int g = 0; g < GMAX; ++g) acc[g][0] = acc[g][1] = 0.f;

  const uint16_t* kb = (const uint16_t*)kv.k;
  const uint16_t* vb = (const uint16_t*)kv.v;
  for (int q0 = p0; q0 < p1; q0 += kThreads) {
    const int cnt = min(kThreads, p1 - q0);
    if ((int)threadIdx.x < cnt) {
      const int pos = q0 + threadIdx.x;
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
      rows_sh[threadIdx.x] = slot >= 0 ? row_elem(kv, b, h, slot, D) : -1;
    } else {
      rows_sh[threadIdx.x] = -1;
    }
    __syncthreads();
    const int n_ch = (cnt + 15) >> 4;
    for (int c0 = wave; c0 < n_ch; c0 += 4 * CH) {
      bf16x8_t Kf[CH][4];
      uint32_t Vw[CH][16];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int c = c0 + 4 * u;
        const int64_t rk = c < n_ch ? rows_sh[c * 16 + n] : -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t w = rk >= 0 ? ld16((const char*)(kb + rk + 8 * (4 * j + g4)))
                                    : u32x4_t{0, 0, 0, 0};
          Kf[u][j] = __builtin_bit_cast(bf16x8_t, w);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int64_t rv = c < n_ch ? rows_sh[c * 16 + t] : -1;
          Vw[u][t] = rv >= 0 ? *(const uint32_t*)(vb + rv + 2 * lane) : 0u;
        }
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int c = c0 + 4 * u;
        if (c < n_ch) {                             // uniform over the wave
        f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf[u][j], Qf[j], S, 0, 0, 0);
        float z[4], cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = rows_sh[c * 16 + 4 * g4 + i] >= 0;
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
        float vf[16][2];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          vf[t][0] = bf16_lo(Vw[u][t]);
          vf[t][1] = bf16_hi(Vw[u][t]);
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
          if (g < G) {
          const float cg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), g));
          // the 16 weights of head g first (scalars read back to back)
          float pg[16];
#pragma unroll
          for (int t = 0; t < 16; ++t)
            pg[t] = __int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(p[t & 3]), g + 16 * (t >> 2)));
          float a0 = acc[g][0] * cg, a1 = acc[g][1] * cg;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            a0 = fmaf(pg[t], vf[t][0], a0);
            a1 = fmaf(pg[t], vf[t][1], a1);
          }
          acc[g][0] = a0;
          acc[g][1] = a1;
          }
        }
        }
      }
    }
    __syncthreads();
  }

  // merge the four waves through LDS
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) continue;
    red[wave][g][2 * lane] = acc[g][0];
    red[wave][g][2 * lane + 1] = acc[g][1];
    if (lane == g) {
      red[wave][g][D] = m_run;
      red[wave][g][D + 1] = l_run;
    }
  }
  __syncthreads();
  const int stride = D + 2;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, j = i - g * D;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][g][D]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float cw = exp2f(red[w][g][D] - mm);
        ll += red[w][g][D + 1] * cw;
        aa += red[w][g][j] * cw;
      }
    }
    float* dst = part + ((((int64_t)b * kv.H + h) * G + g) * n_split + s) * stride;
    dst[j] = aa;
    if (j == 0) {
      dst[D] = mm;
      dst[D + 1] = ll;
    }
  }
}

// out[b][hq][j] = sum_s acc_s[j] 2^(m_s - M) / sum_s l_s 2^(m_s - M)
// Grid (query heads, B, ceil(D / 256)): a workgroup owns 256 dims of one
// (b, query head), a thread one dim, whose values it loads from SG splits at
// a time -- all of them, in flight while the split weights
// are formed (n_split <= 64, D <= 512).
// With zero_hist != nullptr, the first workgroup of the first query head of
// each KV head also zeroes that row's copies of the 4096-bin key histogram
// and, with ctr != nullptr, the row's list counter (ctr[row * kCtrStride]):
// the fused top-k + attention paths leave them for this kernel, which runs
// after every reader.
template <int SG>   // splits whose values are loaded together (32, or 64 for more splits)
__global__ __launch_bounds__(256) void attend_reduce_kernel(const float* part, int n_split, int D,
                                                           int HG, float* out, uint32_t* zero_hist,
                                                           int G, int copies, int32_t* ctr) {
  __shared__ float wts[64];
  __shared__ float inv_l;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int j = blockIdx.z * 256 + threadIdx.x;
  if (zero_hist && hq % G == 0 && blockIdx.z == 0) {
    const int64_t row = (int64_t)b * (HG / G) + hq / G;
    uint4* z = (uint4*)(zero_hist + row * copies * 4096);
    for (int i = threadIdx.x; i < 1024 * copies; i += blockDim.x) z[i] = make_uint4(0u, 0u, 0u, 0u);
    if (ctr && threadIdx.x == 0) ctr[row * kCtrStride] = 0;
  }
  const int stride = D + 2;
  const float* base = part + ((int64_t)b * HG + hq) * n_split * stride;
  float v[SG];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int u = 0; u < SG; ++u)
      v[u] = (s0 + u < n_split && j < D) ? base[(int64_t)(s0 + u) * stride + j] : 0.f;
  };
  load_group(0);
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float ms = s < n_split ? base[(int64_t)s * stride + D] : -INFINITY;
    const float ls = s < n_split ? base[(int64_t)s * stride + D + 1] : 0.f;
    float M = ms;
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float w = (s < n_split && M != -INFINITY) ? exp2f(ms - M) : 0.f;
    float L = ls * w;
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    wts[s] = w;
    if (s == 0) inv_l = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += SG) {
    if (s0) load_group(s0);
#pragma unroll
    for (int u = 0; u < SG; ++u) acc += v[u] * (s0 + u < n_split ? wts[s0 + u] : 0.f);
  }
  if (j < D) out[((int64_t)b * HG + hq) * D + j] = acc * inv_l;
}

template <bool BF16, int NPL>
hipError_t launch_split(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                        const int32_t* lo, const int32_t* hi, float scale_log2, int n_split,
                        float* part, float* out, hipStream_t st) {
  dim3 grid(n_split, kv.H, kv.B);
  const size_t lds = (size_t)4 * G * (kv.d_k + 2) * sizeof(float);
  if (G == 1)
    attend_split_kernel<BF16, NPL, 1><<<grid, kThreads, lds, st>>>(kv, q, G, idx, k, lo, hi, scale_log2, n_split, part, out);
  else if (G == 2)
    attend_split_kernel<BF16, NPL, 2><<<grid, kThreads, lds, st>>>(kv, q, G, idx, k, lo, hi, scale_log2, n_split, part, out);
  else if (G <= 4)
    attend_split_kernel<BF16, NPL, 4><<<grid, kThreads, lds, st>>>(kv, q, G, idx, k, lo, hi, scale_log2, n_split, part, out);
  else if (G <= 8 && NPL == 1)
    attend_split_kernel<BF16, NPL, (NPL == 1 ? 8 : 4)><<<grid, kThreads, lds, st>>>(kv, q, G, idx, k, lo, hi, scale_log2, n_split, part, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int pieces_per_lane(const KvArgs& kv) {
  const int E = kv.bf16 ? 8 : 4;
  if (kv.d_k % (16 * E)) return 0;
  return kv.d_k / (16 * E);
}

}  // namespace

// Splits per row: ~128 selected tokens each (64 at most), and at least enough
// for 256 workgroups when there are few rows (8 KV heads of one sequence:
// 32 splits instead of 4), since the sink / local tokens every split also
// shares are not known on the host.
int attend_num_splits(int k, int rows) {
  int n = std::max(1, std::min(64, (k + 511) / 128));
  if (rows > 0 && (int64_t)rows * n < 256) n = std::min(64, std::max(n, (256 + rows - 1) / rows));
  return n;
}
constexpr int kOneSplitK = 128;   // vector-ALU path: single split, no merge kernel

bool attend_supported(const KvArgs& kv, int G) {
  if (kv.v == nullptr || kv.d_k != kv.d_v) return false;
  const int npl = pieces_per_lane(kv);
  if (npl != 1 && npl != 2) return false;
  if (kv.bf16 && kv.d_k == 128) return G >= 1 && G <= 16;    // matrix-core path
  if (G < 1 || G > 8 || (npl == 2 && G > 4)) return false;
  return true;
}

size_t attend_workspace_bytes(const KvArgs& kv, int G, int k) {
  return (size_t)kv.B * kv.H * G * attend_num_splits(k, kv.B * kv.H) * (kv.d_v + 2) * sizeof(float);
}

hipError_t launch_gather_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                                const int32_t* lo, const int32_t* hi, float scale, float* out,
                                void* ws, size_t ws_bytes, hipStream_t st) {
  const int n_split = attend_num_splits(k, kv.B * kv.H);
  float* part = (float*)ws;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipError_t e;
  const int npl = pieces_per_lane(kv);
  if (kv.bf16 && kv.d_k == 128 && G <= 16) {
    dim3 grid(n_split, kv.H, kv.B);
    const uint16_t* qq = (const uint16_t*)q;
    if (G <= 1)
      attend_mfma_kernel<1><<<grid, kThreads, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part);
    else if (G <= 4)
      attend_mfma_kernel<4><<<grid, kThreads, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part);
    else if (G <= 8)
      attend_mfma_kernel<8><<<grid, kThreads, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part);
    else
      attend_mfma_kernel<16><<<grid, kThreads, 0, st>>>(kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part);
    e = hipGetLastError();
  } else {
    // the vector-ALU path takes a short selection (k <= 128) in one split
    // that writes the output itself: 256 threads have such a row's selected
    // rows in flight at once, and the merge kernel's launch is saved
    const bool one = k <= kOneSplitK;
    const int ns = one ? 1 : n_split;
    float* o1 = one ? out : nullptr;
    if (kv.bf16)
      e = npl == 1 ? launch_split<true, 1>(kv, q, G, idx, k, lo, hi, scale_log2, ns, part, o1, st)
                   : launch_split<true, 2>(kv, q, G, idx, k, lo, hi, scale_log2, ns, part, o1, st);
    else
      e = npl == 1 ? launch_split<false, 1>(kv, q, G, idx, k, lo, hi, scale_log2, ns, part, o1, st)
                   : launch_split<false, 2>(kv, q, G, idx, k, lo, hi, scale_log2, ns, part, o1, st);
    if (one) return e;
  }
  if (e != hipSuccess) return e;
  return launch_attend_reduce(part, n_split, kv.d_v, kv.H * G, kv.B, out, st);
}

hipError_t launch_attend_reduce(const float* part, int n_split, int D, int HG, int B, float* out,
                                hipStream_t st, uint32_t* zero_hist, int G, int copies,
                                int32_t* ctr) {
  if (n_split > 64 || D > 512) return hipErrorInvalidValue;
  dim3 grid(HG, B, (D + 255) / 256);
  if (n_split > 32)
    attend_reduce_kernel<64><<<grid, 256, 0, st>>>(part, n_split, D, HG, out, zero_hist, G, copies,
                                                   ctr);
  else
    attend_reduce_kernel<32><<<grid, 256, 0, st>>>(part, n_split, D, HG, out, zero_hist, G, copies,
                                                   ctr);
  return hipGetLastError();
}

}  // namespace skv
