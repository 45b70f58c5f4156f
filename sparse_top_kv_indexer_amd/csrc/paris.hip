// ParisKV compressed-code retrieval on gfx950: index encoding and the
// retrieval pipeline (collision vote -> bucket top-C -> 4-bit rerank ->
// exact top-k).
//
// Source: ParisKV close-reading (notes on arXiv 2602.07721v3), sections
// 2.2-2.5 (paper Sec. 4.1-4.3, Eqs. (5)-(12), (15), Prop. 4.1).
//
// The method is an approximation, so its floating-point steps are fixed as
// one fp32 operation sequence that this file follows exactly (compiled
// without fp contraction; division is the IEEE-rounded sequence and the
// square root is corrected to round-to-nearest-even, see sqrt_rn):
//   tree sums pair element j with element j + half, halving to one element;
//   |x| = sqrt(tree(x*x)), x^ = x / |x| (0 for a zero row);
//   SRHT: y = x^ * sigma, Walsh-Hadamard butterflies h = 1, 2, ..., 64 with
//   (a, b) -> (a + b, a - b), then y * fp32(1/sqrt(128));
//   subspace b: r = sqrt(tree8(y_b^2)), u = y_b / r; id bit j = [u_j < 0];
//   nibble = [u_j < 0] << 3 | #{thresholds <= |u_j|}; v_j = +-levels[mag];
//   alpha = tree8(v*u); w = (|k| r) / alpha; and for the rerank
//   est = max_g (|q_g| * tree16_b(w_b * tree8_j(v_j * q~_gbj))).
//
// Layout: a key row of d = 128 is held by a 16-lane group, lane j owning
// dims 8j..8j+7 = subspace j, so the per-subspace work stays in registers
// and the cross-subspace tree levels are lane exchanges (xor 8, 4, 2, 1).
#include <math.h>

#include <algorithm>

#include "../../include/sparsekv.h"
#include "skv_device.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kD = 128, kSub = 16, kM = 8, kCent = 256;
constexpr int kVoteBins = 6 * kSub + 1;   // S in [0, 96]
constexpr int kChunk = 2048;              // index entries per vote workgroup
constexpr int kEncPerWG = 2048;           // keys per encode workgroup

struct CodebookArgs {
  float levels[8];
  float thresh[7];
  float c;          // fp32(1 / sqrt(d))
};

struct TierArgs {
  int t_rho;
  int T[6];
};

__device__ __forceinline__ float xor16(float v, int m) { return __shfl_xor(v, m, 64); }

// Correctly rounded fp32 square root of x >= 0.  The hardware square root is
// within one ulp; the neighbour that is nearest to sqrt(x) is picked by
// comparing x with the squared midpoints between neighbours, which are exact
// in double (a 25-bit midpoint squares to at most 50 bits) and never equal x.
__device__ __forceinline__ float sqrt_rn(float x) {
  if (!(x > 0.f)) return x == 0.f ? 0.f : __builtin_nanf("");
  float f = (float)__builtin_sqrt((double)x);
  const double d = (double)x;
  const uint32_t fb = __float_as_uint(f);
  const float f_dn = __uint_as_float(fb - 1u), f_up = __uint_as_float(fb + 1u);
  const double m_lo = 0.5 * ((double)f_dn + (double)f);
  const double m_hi = 0.5 * ((double)f + (double)f_up);
  if (d < m_lo * m_lo) f = f_dn;
  else if (d > m_hi * m_hi) f = f_up;
  return f;
}

__device__ __forceinline__ float tree8(const float* a) {
  const float b0 = a[0] + a[4], b1 = a[1] + a[5], b2 = a[2] + a[6], b3 = a[3] + a[7];
  const float c0 = b0 + b2, c1 = b1 + b3;
  return c0 + c1;
}

// Normalise and rotate one d = 128 row held by a 16-lane group (lane j: dims
// 8j..8j+7).  Returns |x|; x becomes R x^.
__device__ __forceinline__ float rotate_row(float* x, int j, const float* sg, float c) {
  float sq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sq[e] = x[e] * x[e];
  // tree over 128: dims d and d + 64 live in lanes j and j ^ 8, etc.
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = sq[e] + xor16(sq[e], m);
  const float nrm = sqrt_rn(tree8(sq));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = nrm > 0.f ? __fdiv_rn(x[e], nrm) : 0.f;
    x[e] = sg[e] > 0.f ? x[e] : -x[e];
  }
  float a, b;
  // h = 1
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    a = x[e]; b = x[e + 1]; x[e] = a + b; x[e + 1] = a - b;
  }
  // h = 2
#pragma unroll
  for (int e = 0; e < 8; e += 4)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      a = x[e + f]; b = x[e + f + 2]; x[e + f] = a + b; x[e + f + 2] = a - b;
    }
  // h = 4
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a = x[f]; b = x[f + 4]; x[f] = a + b; x[f + 4] = a - b;
  }
  // h = 8, 16, 32, 64: partner lane j ^ 1, 2, 4, 8
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = xor16(x[e], m);
      x[e] = (j & m) ? (p - x[e]) : (x[e] + p);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] * c;
  return nrm;
}

__device__ __forceinline__ void load_row8(const KvArgs& kv, int b, int h, int t, int j,
                                          float* x) {
  const int64_t slot = slot_of(kv, b, t);
  if (slot < 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    return;
  }
  const u32x4_t wv = *(const u32x4_t*)((const uint16_t*)kv.k + row_elem(kv, b, h, slot, kD) + 8 * j);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(wv[e]);
    x[2 * e + 1] = bf16_hi(wv[e]);
  }
}

// ------------------------------------------------------------------ encode --
__global__ __launch_bounds__(256) void encode_kernel(KvArgs kv, int b, int t0, int n_keys, int n0,
                                                     int cap, const int8_t* signs, CodebookArgs cb,
                                                     uint8_t* ids, uint8_t* codes, float* w,
                                                     int32_t* hist, int32_t* pos) {
  __shared__ uint32_t lh[kSub * kCent];
  const int h = blockIdx.y;
  const int j = threadIdx.x & 15, grp = threadIdx.x >> 4;
  for (int i = threadIdx.x; i < kSub * kCent; i += 256) lh[i] = 0u;
  __syncthreads();
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = (float)signs[8 * j + e];
  const int k0 = blockIdx.x * kEncPerWG, k1 = min(n_keys, k0 + kEncPerWG);
  for (int key = k0 + grp; key < k1; key += 16) {
    const int t = t0 + key;
    float x[8];
    load_row8(kv, b, h, t, j, x);
    const float nrm = rotate_row(x, j, sg, cb.c);
    // subspace j
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = x[e] * x[e];
    const float r = sqrt_rn(tree8(a));
    uint32_t id = 0u, code = 0u;
    float vu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = r > 0.f ? __fdiv_rn(x[e], r) : 0.f;
      const bool ng = u < 0.f;
      const float au = fabsf(u);
      uint32_t mag = 0u;
      float lv = cb.levels[0];
#pragma unroll
      for (int i = 0; i < 7; ++i)
        if (au >= cb.thresh[i]) {
          mag = i + 1;
          lv = cb.levels[i + 1];
        }
      id |= (uint32_t)ng << e;
      code |= (((uint32_t)ng << 3) | mag) << (4 * e);
      const float v = ng ? -lv : lv;
      vu[e] = v * u;
    }
    const float alpha = tree8(vu);
    const float wv = r > 0.f ? __fdiv_rn(nrm * r, alpha) : 0.f;
    const int64_t ent = (int64_t)h * cap + n0 + key;
    ids[ent * kSub + j] = (uint8_t)id;
    ((uint32_t*)codes)[ent * kSub + j] = code;
    w[ent * kSub + j] = wv;
    atomicAdd(&lh[j * kCent + id], 1u);
    if (h == 0 && j == 0) pos[n0 + key] = t;
  }
  __syncthreads();
  int32_t* gh = hist + (int64_t)h * kSub * kCent;
  for (int i = threadIdx.x; i < kSub * kCent; i += 256)
    if (lh[i]) atomicAdd(&gh[i], (int32_t)lh[i]);
}

// --------------------------------------------------------------- query LUT --
// One workgroup per query head: rotate the query, rank the 256 centroids of
// each subspace by similarity (ties: lower id) and assign tier weights from
// the exclusive prefix counts of the index histogram.
__global__ __launch_bounds__(256) void query_lut_kernel(const uint16_t* q, int G,
                                                        const int8_t* signs, float c,
                                                        const int32_t* hist, TierArgs ta,
                                                        float* qt_out, float* qn_out,
                                                        uint8_t* lut) {
  __shared__ float qt[kD];
  __shared__ float sims[kCent];
  __shared__ int cnt_sorted[kCent];
  __shared__ int wsum[4];
  const int hq = blockIdx.x, h = hq / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 16) {
    const int j = tid;
    float x[8], sg[8];
    const u32x4_t wv = *(const u32x4_t*)(q + (int64_t)hq * kD + 8 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(wv[e]);
      x[2 * e + 1] = bf16_hi(wv[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)signs[8 * j + e];
    const float nrm = rotate_row(x, j, sg, c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qt[8 * j + e] = x[e];
      qt_out[(int64_t)hq * kD + 8 * j + e] = x[e];
    }
    if (j == 0) qn_out[hq] = nrm;
  }
  __syncthreads();
  const int cid = tid;   // centroid of this thread
  for (int sb = 0; sb < kSub; ++sb) {
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = qt[8 * sb + e];
      pr[e] = ((cid >> e) & 1) ? -v : v;
    }
    const float sim = tree8(pr);
    sims[cid] = sim;
    __syncthreads();
    int rank = 0;
    for (int c2 = 0; c2 < kCent; ++c2) {
      const float s2 = sims[c2];
      rank += (s2 > sim) || (s2 == sim && c2 < cid);
    }
    const int cnt = hist[((int64_t)h * kSub + sb) * kCent + cid];
    cnt_sorted[rank] = cnt;
    __syncthreads();
    // exclusive prefix over the ranked order
    const int v = cnt_sorted[tid];
    const int ex = wave_excl_scan(v, lane);
    if (lane == 63) wsum[wave] = ex + v;
    __syncthreads();
    int before = ex;
    for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
    cnt_sorted[tid] = before;           // now P at ranked position tid
    __syncthreads();
    const int P = cnt_sorted[rank];
    int wt = 0;
    if (P < ta.t_rho) {
      int ell = 0;
#pragma unroll
      for (int i = 0; i < 6; ++i) ell += ta.T[i] <= P;
      wt = 6 - ell;
    }
    lut[((int64_t)hq * kSub + sb) * kCent + cid] = (uint8_t)wt;
    __syncthreads();
  }
}

// -------------------------------------------------------------------- vote --
// S_i = max_g sum_b LUT_g[b][id_ib]: the G <= 4 query heads' tier bytes are
// packed into one u32 per (subspace, centroid), so one LDS lookup per
// subspace serves the whole group (a byte never exceeds 96).  Each
// workgroup also histograms its S values (32 bank-spread copies in LDS).
__global__ __launch_bounds__(256) void vote_kernel(const uint8_t* ids, int cap, int n, int G,
                                                   const uint8_t* lut, uint8_t* votes,
                                                   int32_t* chunk_hist, int n_chunks) {
  __shared__ uint32_t lut4[kSub * kCent];
  __shared__ uint32_t vh[kVoteBins * 32];
  const int h = blockIdx.y, chunk = blockIdx.x;
  for (int i = threadIdx.x; i < kSub * kCent; i += 256) {
    uint32_t p = 0u;
    for (int g = 0; g < G; ++g) p |= (uint32_t)lut[(int64_t)(h * G + g) * kSub * kCent + i] << (8 * g);
    lut4[i] = p;
  }
  for (int i = threadIdx.x; i < kVoteBins * 32; i += 256) vh[i] = 0u;
  __syncthreads();
  const int copy = threadIdx.x & 31;
  const int i0 = chunk * kChunk;
  const u32x4_t* idrow = (const u32x4_t*)(ids + (int64_t)h * cap * kSub);
  constexpr int U = kChunk / 256;
  u32x4_t idv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * 256 + threadIdx.x;
    idv[u] = i < n ? idrow[i] : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * 256 + threadIdx.x;
    if (i >= n) continue;
    uint32_t acc = 0u;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int sb = q4 * 4 + bb;
        acc += lut4[sb * kCent + ((idv[u][q4] >> (8 * bb)) & 0xffu)];
      }
    uint32_t S = acc & 0xffu;
    for (int g = 1; g < G; ++g) S = max(S, (acc >> (8 * g)) & 0xffu);
    votes[(int64_t)h * n + i] = (uint8_t)S;
    atomicAdd(&vh[S * 32 + copy], 1u);
  }
  __syncthreads();
  for (int v = threadIdx.x; v < kVoteBins; v += 256) {
    uint32_t sum = 0u;
    for (int cp = 0; cp < 32; ++cp) sum += vh[v * 32 + cp];
    chunk_hist[((int64_t)h * n_chunks + chunk) * kVoteBins + v] = (int32_t)sum;
  }
}

// -------------------------------------------------------------------- scan --
// One workgroup per KV head: the vote threshold s* and, per chunk, the
// output offset of its candidates and how many S == s* entries it takes
// (lowest entries first).
__global__ __launch_bounds__(256) void cand_scan_kernel(const int32_t* chunk_hist, int n_chunks,
                                                        int C, int32_t* chunk_off,
                                                        int32_t* chunk_take, int32_t* win,
                                                        int32_t* sstar) {
  __shared__ int tot[kVoteBins];
  __shared__ int s_star, s_need;
  __shared__ int wsum[4];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* ch = chunk_hist + (int64_t)h * n_chunks * kVoteBins;
  for (int v = tid; v < kVoteBins; v += 256) {
    int s = 0;
    for (int c = 0; c < n_chunks; ++c) s += ch[(int64_t)c * kVoteBins + v];
    tot[v] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int above = 0, star = -1, need = 0;
    for (int v = kVoteBins - 1; v >= 0; --v) {
      if (above + tot[v] >= C) {
        star = v;
        need = C - above;
        break;
      }
      above += tot[v];
    }
    s_star = star;      // -1: every entry is a candidate (C >= n)
    s_need = need;
    sstar[h] = star;
    if (h == 0) {
      win[0] = 0;
      win[1] = C;
    }
  }
  __syncthreads();
  const int star = s_star, need = s_need;
  // per-chunk counts above s* and equal to s*, exclusive scans over chunks
  int run_gt = 0, run_eq = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += 256) {
    const int c = c0 + tid;
    int gt = 0, eq = 0;
    if (c < n_chunks) {
      for (int v = 0; v < kVoteBins; ++v) {
        const int x = ch[(int64_t)c * kVoteBins + v];
        if (star < 0 || v > star) gt += x;
        else if (v == star) eq += x;
      }
    }
    const int egt = wave_excl_scan(gt, lane), eeq = wave_excl_scan(eq, lane);
    __syncthreads();
    if (lane == 63) wsum[wave] = egt + gt;
    __syncthreads();
    int bgt = egt;
    int tgt = 0;
    for (int w2 = 0; w2 < 4; ++w2) {
      if (w2 < wave) bgt += wsum[w2];
      tgt += wsum[w2];
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = eeq + eq;
    __syncthreads();
    int beq = eeq;
    int teq = 0;
    for (int w2 = 0; w2 < 4; ++w2) {
      if (w2 < wave) beq += wsum[w2];
      teq += wsum[w2];
    }
    if (c < n_chunks) {
      const int eq_before = run_eq + beq;
      const int take = max(0, min(eq, need - eq_before));
      chunk_off[(int64_t)h * n_chunks + c] = run_gt + bgt + min(eq_before, need);
      chunk_take[(int64_t)h * n_chunks + c] = star < 0 ? 0 : take;
    }
    run_gt += tgt;
    run_eq += teq;
    __syncthreads();
  }
}

// ------------------------------------------------------------------ compact --
// Ordered compaction of each chunk's candidates: S > s*, or S == s* among the
// chunk's first `take` such entries.
__global__ __launch_bounds__(256) void cand_write_kernel(const uint8_t* votes, int n, int n_chunks,
                                                         int C, const int32_t* sstar,
                                                         const int32_t* chunk_off,
                                                         const int32_t* chunk_take,
                                                         int32_t* cand) {
  __shared__ int wa[4], we[4];
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int s_star;
  if (threadIdx.x == 0) s_star = sstar[h];
  __syncthreads();
  const int star = s_star;
  const int off = chunk_off[(int64_t)h * n_chunks + chunk];
  const int take = chunk_take[(int64_t)h * n_chunks + chunk];
  constexpr int kSeg = kChunk / 4;   // entries per wave
  const int i0 = chunk * kChunk + wave * kSeg;
  const uint8_t* vr = votes + (int64_t)h * n;
  int sv[kSeg / 64];
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    const int i = i0 + u * 64 + lane;
    sv[u] = i < n ? (int)vr[i] : -1;
  }
  int ca = 0, ce = 0;
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    ca += __popcll(__ballot(sv[u] >= 0 && (star < 0 || sv[u] > star)));
    ce += __popcll(__ballot(star >= 0 && sv[u] == star));
  }
  if (lane == 0) {
    wa[wave] = ca;
    we[wave] = ce;
  }
  __syncthreads();
  int oa = 0, oe = 0;
  for (int v = 0; v < wave; ++v) {
    oa += wa[v];
    oe += we[v];
  }
  const uint64_t lt = lanemask_lt(lane);
  int32_t* crow = cand + (int64_t)h * C;
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    const bool is_gt = sv[u] >= 0 && (star < 0 || sv[u] > star);
    const bool is_eq = star >= 0 && sv[u] == star;
    const uint64_t ba = __ballot(is_gt), be = __ballot(is_eq);
    const int a_before = oa + __popcll(ba & lt);
    const int e_before = oe + __popcll(be & lt);
    const bool sel = is_gt || (is_eq && e_before < take);
    const int dst = off + a_before + min(e_before, take);
    if (sel && dst < C) crow[dst] = i0 + u * 64 + lane;
    oa += __popcll(ba);
    oe += __popcll(be);
  }
}

// ------------------------------------------------------------------ rerank --
// est_i = max_g fl(|q_g| * tree16_b fl(w_ib * tree8_j fl(v_ibj * q~_gbj)));
// a 16-lane group per candidate, lane b = subspace b.
__global__ __launch_bounds__(256) void rerank_kernel(const uint8_t* codes, const float* w, int cap,
                                                     int n, const int32_t* cand, int C, int G,
                                                     const float* qt, const float* qn,
                                                     CodebookArgs cb, float* est) {
  const int h = blockIdx.y;
  const int j = threadIdx.x & 15, grp = threadIdx.x >> 4;
  float qv[4][8], qs[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int hq = h * G + min(g, G - 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[g][e] = qt[(int64_t)hq * kD + 8 * j + e];
    qs[g] = qn[hq];
  }
  const int per_wg = 64;
  const int c0 = blockIdx.x * per_wg;
  for (int ci = c0 + grp; ci < min(C, c0 + per_wg); ci += 16) {
    const int64_t ent = (int64_t)h * cap + min(max(cand[(int64_t)h * C + ci], 0), n - 1);
    const uint32_t code = ((const uint32_t*)codes)[ent * kSub + j];
    const float wb = w[ent * kSub + j];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t nib = (code >> (4 * e)) & 0xfu;
      const uint32_t mag = nib & 7u;
      float lv = cb.levels[0];
#pragma unroll
      for (int i = 1; i < 8; ++i)
        if (mag == (uint32_t)i) lv = cb.levels[i];
      v[e] = (nib & 8u) ? -lv : lv;
    }
    float best = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g >= G) break;
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = v[e] * qv[g][e];
      float x = wb * tree8(pr);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) x = x + xor16(x, m);
      const float e_g = qs[g] * x;
      best = g == 0 ? e_g : fmaxf(best, e_g);
    }
    if (j == 0) est[(int64_t)h * C + ci] = best;
  }
}

// An empty index retrieves nothing.
__global__ void empty_kernel(int k_final, int32_t* idx, int32_t* n_cand) {
  const int h = blockIdx.x;
  for (int i = threadIdx.x; i < k_final; i += blockDim.x) idx[(int64_t)h * k_final + i] = -1;
  if (threadIdx.x == 0) n_cand[h] = 0;
}

// --------------------------------------------------------------------- map --
__global__ void map_kernel(const int32_t* tk_idx, const int32_t* tk_cnt, const int32_t* cand,
                           int C, const int32_t* pos, int k_final, int32_t* idx,
                           int32_t* n_cand) {
  const int h = blockIdx.x;
  const int cnt = tk_cnt[h];
  for (int i = threadIdx.x; i < k_final; i += blockDim.x) {
    int v = -1;
    if (i < cnt) {
      const int p = tk_idx[(int64_t)h * k_final + i];
      v = pos[cand[(int64_t)h * C + p]];
    }
    idx[(int64_t)h * k_final + i] = v;
  }
  if (threadIdx.x == 0) n_cand[h] = cnt;
}

// workspace of a retrieval; the top-k part comes first (zero-filled region)
struct RetrieveWs {
  void* topk;
  uint8_t* lut;       // [Hq][16][256]
  float* qt;          // [Hq][128]
  float* qn;          // [Hq]
  uint8_t* votes;     // [H][n]
  int32_t* chunk_hist;  // [H][n_chunks][97]
  int32_t* chunk_off;   // [H][n_chunks]
  int32_t* chunk_take;  // [H][n_chunks]
  int32_t* win;       // [2]: top-k window over the candidates
  int32_t* sstar;     // [H]: vote threshold
  int32_t* cand;      // [H][C]
  float* est;         // [H][C]
  int32_t* tk_idx;    // [H][k_final]
  int32_t* tk_cnt;    // [H]

  static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t layout(RetrieveWs* w, char* base, int H, int G, int n, int C, int k_final) {
    const int n_chunks = (n + kChunk - 1) / kChunk;
    const int Hq = H * G;
    size_t o = 0;
    auto take = [&](size_t bytes) {
      char* p = base ? base + o : nullptr;
      o += al(bytes);
      return p;
    };
    void* tk = take(topk_workspace_bytes(H, std::max(C, 1)));
    uint8_t* lut = (uint8_t*)take((size_t)Hq * kSub * kCent);
    float* qt = (float*)take((size_t)Hq * kD * 4);
    float* qn = (float*)take((size_t)Hq * 4);
    uint8_t* votes = (uint8_t*)take((size_t)H * n);
    int32_t* chh = (int32_t*)take((size_t)H * n_chunks * kVoteBins * 4);
    int32_t* cho = (int32_t*)take((size_t)H * n_chunks * 4);
    int32_t* cht = (int32_t*)take((size_t)H * n_chunks * 4);
    int32_t* win = (int32_t*)take(8);
    int32_t* sst = (int32_t*)take((size_t)H * 4);
    int32_t* cand = (int32_t*)take((size_t)H * C * 4);
    float* est = (float*)take((size_t)H * C * 4);
    int32_t* tki = (int32_t*)take((size_t)H * k_final * 4);
    int32_t* tkc = (int32_t*)take((size_t)H * 4);
    if (w) {
      w->topk = tk;
      w->lut = lut;
      w->qt = qt;
      w->qn = qn;
      w->votes = votes;
      w->chunk_hist = chh;
      w->chunk_off = cho;
      w->chunk_take = cht;
      w->win = win;
      w->sstar = sst;
      w->cand = cand;
      w->est = est;
      w->tk_idx = tki;
      w->tk_cnt = tkc;
    }
    return o;
  }
};

int n_candidates(int n, double beta) {
  const double c = ceil(beta * (double)n);
  return (int)std::min<double>(n, std::max<double>(c, 0.0));
}

CodebookArgs cb_args(const skv_codebook* cb) {
  CodebookArgs a;
  for (int i = 0; i < 8; ++i) a.levels[i] = cb->levels[i];
  for (int i = 0; i < 7; ++i) a.thresh[i] = cb->thresh[i];
  a.c = (float)(1.0 / sqrt((double)cb->d));
  return a;
}

bool codebook_ok(const skv_codebook* cb) {
  if (!cb || !cb->signs) return false;
  if (cb->d != kD || cb->n_sub != kSub || cb->m != kM) return false;
  for (int i = 0; i < 6; ++i)
    if (!(cb->thresh[i] <= cb->thresh[i + 1])) return false;
  return true;
}

bool index_ok(const skv_index* ix) {
  return ix && ix->ids && ix->codes && ix->w && ix->hist && ix->pos && ix->H >= 1 &&
         ix->cap >= 0 && ix->n >= 0 && ix->n <= ix->cap;
}

}  // namespace

}  // namespace skv

using namespace skv;

extern "C" {

skv_status sparsekv_encode(const skv_codebook* cb, const skv_kv* kv, int32_t b, int32_t t0,
                           int32_t t1, skv_index* index, hipStream_t stream) {
  if (!cb || !kv || !index) return SKV_EINVAL;
  if (!codebook_ok(cb) || !index_ok(index)) return SKV_EINVAL;
  if (!kv->k || !kv->seq_len || kv->dtype != SKV_BF16 || kv->d_k != kD) return SKV_EUNSUPPORTED;
  if (kv->token_table) return SKV_EUNSUPPORTED;
  if (kv->H != index->H || b < 0 || b >= kv->B || t0 < 0 || t1 < t0 || t1 > kv->L_max)
    return SKV_EINVAL;
  const int n_keys = t1 - t0;
  if (index->n + n_keys > index->cap) return SKV_EINVAL;
  if (n_keys == 0) return SKV_OK;
  KvArgs a;
  a.k = kv->k;
  a.v = kv->v;
  a.bf16 = 1;
  a.B = kv->B;
  a.H = kv->H;
  a.d_k = kv->d_k;
  a.d_v = kv->d_v;
  a.block = kv->block;
  a.L_max = kv->L_max;
  a.block_table = kv->block_table;
  a.token_table = nullptr;
  a.seq_len = kv->seq_len;
  dim3 grid((n_keys + kEncPerWG - 1) / kEncPerWG, kv->H);
  encode_kernel<<<grid, 256, 0, stream>>>(a, b, t0, n_keys, index->n, index->cap, cb->signs,
                                          cb_args(cb), index->ids, index->codes, index->w,
                                          index->hist, index->pos);
  if (hipGetLastError() != hipSuccess) return SKV_ELAUNCH;
  index->n += n_keys;
  return SKV_OK;
}

size_t sparsekv_retrieve_workspace_size(const skv_index* index, int32_t G, double beta,
                                        int32_t k_final) {
  if (!index || index->H < 1 || index->n < 0 || G < 1 || k_final < 1 || !(beta > 0)) return 0;
  const int C = n_candidates(index->n, beta);
  return RetrieveWs::layout(nullptr, nullptr, index->H, G, index->n, std::max(C, 1), k_final);
}

skv_status sparsekv_retrieve(const skv_codebook* cb, const skv_index* index, const void* q,
                             int32_t G, double rho, double beta, int32_t k_final, int32_t* idx,
                             int32_t* n_cand, const skv_retrieve_trace* trace, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!codebook_ok(cb) || !index_ok(index) || !q || !idx || !n_cand) return SKV_EINVAL;
  if (G < 1 || k_final < 1 || !(beta > 0) || !(rho >= beta) || !(rho <= 1.0) || !(beta <= 1.0))
    return SKV_EINVAL;
  if (G > 4) return SKV_EUNSUPPORTED;
  const int H = index->H, n = index->n;
  if (n == 0) {
    empty_kernel<<<H, 128, 0, stream>>>(k_final, idx, n_cand);
    return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
  }
  const int C = std::max(1, n_candidates(n, beta));
  const size_t need = sparsekv_retrieve_workspace_size(index, G, beta, k_final);
  if (!ws || ws_bytes < need) return SKV_EWORKSPACE;
  if (!topk_supported(C)) return SKV_EUNSUPPORTED;
  RetrieveWs w;
  RetrieveWs::layout(&w, (char*)ws, H, G, n, C, k_final);
  uint8_t* votes = (trace && trace->votes) ? trace->votes : w.votes;
  int32_t* cand = (trace && trace->cand) ? trace->cand : w.cand;
  float* est = (trace && trace->est) ? trace->est : w.est;
  const int n_chunks = std::max(1, (n + kChunk - 1) / kChunk);

  TierArgs ta;
  ta.t_rho = (int)ceil(rho * (double)n);
  const double fr[6] = {0.05, 0.15, 0.30, 0.50, 0.75, 1.0};
  for (int i = 0; i < 6; ++i) ta.T[i] = (int)ceil(fr[i] * (double)ta.t_rho);
  const CodebookArgs ca = cb_args(cb);

  query_lut_kernel<<<H * G, 256, 0, stream>>>((const uint16_t*)q, G, cb->signs, ca.c, index->hist,
                                              ta, w.qt, w.qn, w.lut);
  vote_kernel<<<dim3(n_chunks, H), 256, 0, stream>>>(index->ids, index->cap, n, G, w.lut, votes,
                                                     w.chunk_hist, n_chunks);
  cand_scan_kernel<<<H, 256, 0, stream>>>(w.chunk_hist, n_chunks, C, w.chunk_off, w.chunk_take,
                                          w.win, w.sstar);
  cand_write_kernel<<<dim3(n_chunks, H), 256, 0, stream>>>(votes, n, n_chunks, C, w.sstar,
                                                           w.chunk_off, w.chunk_take, cand);
  rerank_kernel<<<dim3((C + 63) / 64, H), 256, 0, stream>>>(index->codes, index->w, index->cap,
                                                            n, cand, C, G, w.qt, w.qn, ca, est);
  hipError_t e = launch_topk(est, H, H, C, w.win, w.win + 1, k_final, w.tk_idx, w.tk_cnt, w.topk,
                             false, stream);
  if (e != hipSuccess) return SKV_ELAUNCH;
  map_kernel<<<H, 128, 0, stream>>>(w.tk_idx, w.tk_cnt, cand, C, index->pos, k_final, idx, n_cand);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // extern "C"
