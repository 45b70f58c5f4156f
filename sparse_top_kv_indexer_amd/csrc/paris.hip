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
#include "skv_rowsel.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kD = 128, kSub = 16, kM = 8, kCent = 256;
constexpr int kVoteBins = 6 * kSub + 1;   // S in [0, 96]
constexpr int kGe = kVoteBins + 1;        // suffix counts #(S >= v), v = 0..97
constexpr int kChunk = 8192;              // index entries per vote / compaction workgroup
constexpr int kEncPerWG = 2048;           // most keys per encode workgroup

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
// Grid (ceil(n_keys / per_wg), H): a workgroup encodes per_wg keys of one
// head, 16 lanes per key.  Large appends (per_wg = 2048) count centroid ids
// in LDS and add the counts once per workgroup; small ones (an Update Buffer
// flush: per_wg <= 64, many workgroups with a few keys each) add each key's
// 16 ids straight to the index histogram.
__global__ __launch_bounds__(256) void encode_kernel(KvArgs kv, int b, int t0, int n_keys, int n0,
                                                     int cap, int per_wg, const int8_t* signs,
                                                     CodebookArgs cb, uint8_t* ids, uint32_t* cw,
                                                     int32_t* hist, int32_t* pos) {
  __shared__ uint32_t lh[kSub * kCent];
  const int h = blockIdx.y;
  const int j = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const bool direct = per_wg <= 64;
  int32_t* gh = hist + (int64_t)h * kSub * kCent;
  if (!direct) {
    for (int i = threadIdx.x; i < kSub * kCent; i += 256) lh[i] = 0u;
    __syncthreads();
  }
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = (float)signs[8 * j + e];
  const int k0 = blockIdx.x * per_wg, k1 = min(n_keys, k0 + per_wg);
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
    ((uint2*)cw)[ent * kSub + j] = make_uint2(code, __float_as_uint(wv));
    if (direct)
      atomicAdd(&gh[j * kCent + id], 1);
    else
      atomicAdd(&lh[j * kCent + id], 1u);
    if (h == 0 && j == 0) pos[n0 + key] = t;
  }
  if (direct) return;
  __syncthreads();
  for (int i = threadIdx.x; i < kSub * kCent; i += 256)
    if (lh[i]) atomicAdd(&gh[i], (int32_t)lh[i]);
}

// --------------------------------------------------------------- query LUT --
// Grid (16 subspaces, H KV heads, 4), 256 threads: workgroup (b, h, g) serves
// query head h G + g in subspace b, one centroid per thread.  It rotates the
// query (16 lanes) and keeps subspace b, ranks the 256 centroids by
// similarity (ties: lower id), walks the ranking with the exclusive prefix
// count of the index histogram and assigns the tier weights.  A rank is a
// count of larger keys, the key being the similarity's order-preserving bits
// (-0 = +0) above 255 - id, so ties need no second compare.  The LUT word of
// (h, b, centroid) packs the G heads' weights into its bytes (byte g written
// by workgroup g; 0 in bytes G..3), so the vote takes one lookup per subspace
// for the whole group.
__global__ __launch_bounds__(256) void query_lut_kernel(const uint16_t* q, int G,
                                                        const int8_t* signs, float c,
                                                        const int32_t* hist, TierArgs ta,
                                                        float* qt_out, float* qn_out,
                                                        uint8_t* lut) {
  __shared__ float qsub[8];
  __shared__ __align__(16) uint64_t keys[kCent];
  __shared__ int ranked[kCent];
  __shared__ int wsum[4];
  const int sb = blockIdx.x, h = blockIdx.y, g = blockIdx.z;
  const int cid = threadIdx.x, lane = cid & 63, wave = cid >> 6;
  uint8_t* dst = lut + (((int64_t)h * kSub + sb) * kCent + cid) * 4 + g;
  if (g >= G) {   // uniform over the workgroup
    *dst = 0;
    return;
  }
  const int hq = h * G + g;
  const int cnt = hist[((int64_t)h * kSub + sb) * kCent + cid];
  if (cid < 16) {
    const int j = cid;
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
    if (j == sb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qsub[e] = x[e];
    }
    if (sb == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qt_out[(int64_t)hq * kD + 8 * j + e] = x[e];
      if (j == 0) qn_out[hq] = nrm;
    }
  }
  __syncthreads();
  float pr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = qsub[e];
    pr[e] = ((cid >> e) & 1) ? -v : v;
  }
  uint32_t u = __float_as_uint(tree8(pr));
  if (u == 0x80000000u) u = 0u;   // -0 ranks with +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint64_t key = ((uint64_t)ord << 8) | (uint64_t)(255 - cid);
  keys[cid] = key;
  lds_barrier();
  int rank = 0;
  const ulonglong2* k2 = (const ulonglong2*)keys;
#pragma unroll 8
  for (int i = 0; i < kCent / 2; ++i) {
    const ulonglong2 kk = k2[i];
    rank += kk.x > key;
    rank += kk.y > key;
  }
  ranked[rank] = cnt;
  lds_barrier();
  // exclusive prefix of the counts in ranked order
  const int v = ranked[cid];
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  lds_barrier();
  int before = incl - v;
  for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
  ranked[cid] = before;   // now P at ranked position cid
  lds_barrier();
  const int P = ranked[rank];
  int wt = 0;
  if (P < ta.t_rho) {
    int ell = 0;
#pragma unroll
    for (int i = 0; i < 6; ++i) ell += ta.T[i] <= P;
    wt = 6 - ell;
  }
  *dst = (uint8_t)wt;
}

// -------------------------------------------------------------------- vote --
// Grid (n_chunks, H), 256 threads, kChunk entries per workgroup:
// S_i = max_g sum_b LUT_g[b][id_ib] from one packed-LUT lookup per subspace
// into votes [H][ldv] (ldv: n rounded up to 16 bytes; also into the caller's
// [H][n] trace array when one is given)
// (a byte never exceeds 96, so the four sums never carry into each other).
// The workgroup histograms its S values (32 bank-spread copies in LDS) and
// writes the suffix counts ge[v] = #(S >= v), v = 0..97, of its chunk, which
// it also adds into the head's totals.  A thread takes 4 entries per round
// (8 rounds), the next round's loads in flight during the lookups; the ids
// are read once, with non-temporal loads (each wave load is 1 KB of whole
// lines; plain loads: retrieval 80.2 against 78 us).  8 entries
// per round took 40 us against 37 us on 8 x 1M entries, and spreading a
// wave's lookups over the 16 tables (ids rotated per lane so that lanes hit
// different banks) cost more ALU than the bank conflicts it saved (41-52 us).
__global__ __launch_bounds__(256) void vote_kernel(const uint8_t* ids, int cap, int n,
                                                   const uint32_t* lut, uint8_t* votes, int ldv,
                                                   uint8_t* votes_trace, int32_t* chunk_ge,
                                                   int n_chunks, int32_t* tot_ge) {
  __shared__ __align__(16) uint32_t lut4[kSub * kCent];
  __shared__ uint32_t vh[kVoteBins * 32];
  __shared__ int cnt[128];
  const int h = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const uint4* lsrc = (const uint4*)(lut + (int64_t)h * kSub * kCent);
  uint4 lv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) lv[u] = lsrc[u * 256 + tid];
  const int i0 = chunk * kChunk;
  const u32x4_t* idrow = (const u32x4_t*)(ids + (int64_t)h * cap * kSub);
  constexpr int U = 4;                        // entries per thread per round
  constexpr int R = kChunk / (256 * U);       // rounds
  u32x4_t cur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * 256 + tid;
    cur[u] = i < n ? __builtin_nontemporal_load(idrow + i) : u32x4_t{0, 0, 0, 0};
  }
  for (int i = tid; i < kVoteBins * 32; i += 256) vh[i] = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) ((uint4*)lut4)[u * 256 + tid] = lv[u];
  lds_barrier();
  const int copy = tid & 31;
  uint8_t* vrow = votes + (int64_t)h * ldv;
  uint8_t* trow = votes_trace ? votes_trace + (int64_t)h * n : nullptr;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    u32x4_t nxt[U];
    if (r + 1 < R) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + ((r + 1) * U + u) * 256 + tid;
        nxt[u] = i < n ? __builtin_nontemporal_load(idrow + i) : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + (r * U + u) * 256 + tid;
      if (i >= n) continue;
      uint32_t acc = 0u;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
          acc += lut4[(q4 * 4 + bb) * kCent + ((cur[u][q4] >> (8 * bb)) & 0xffu)];
      const uint32_t S = max(max(acc & 0xffu, (acc >> 8) & 0xffu),
                             max((acc >> 16) & 0xffu, acc >> 24));
      vrow[i] = (uint8_t)S;
      if (trow) trow[i] = (uint8_t)S;
      atomicAdd(&vh[S * 32 + copy], 1u);
    }
    if (r + 1 < R) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
  lds_barrier();
  if (tid < 128) {
    int s = 0;
    if (tid < kVoteBins) {
#pragma unroll 8
      for (int k = 0; k < 32; ++k) s += (int)vh[tid * 32 + ((k + tid) & 31)];
    }
    cnt[tid] = s;
  }
  lds_barrier();
  if (tid < 64) {
    const int c0 = cnt[2 * tid], c1 = cnt[2 * tid + 1];
    const int incl = wave_incl_scan(c0 + c1);
    const int ge0 = wave_total(incl) - (incl - c0 - c1), ge1 = ge0 - c0;
    int32_t* out = chunk_ge + ((int64_t)h * n_chunks + chunk) * kGe;
    int32_t* tot = tot_ge + (int64_t)h * kGe;
    if (2 * tid < kGe) {
      out[2 * tid] = ge0;
      if (ge0) atomicAdd(&tot[2 * tid], ge0);
    }
    if (2 * tid + 1 < kGe) {
      out[2 * tid + 1] = ge1;
      if (ge1) atomicAdd(&tot[2 * tid + 1], ge1);
    }
  }
}

// ------------------------------------------------------------------ compact --
// Grid (n_chunks, H), 256 threads.  The vote threshold s* of head h is the
// largest v with #(S >= v) >= C; the candidates are the entries with S > s*
// and the first need = C - #(S > s*) entries with S == s*, in entry order.
// Each workgroup finds s* from the head's totals, counts the candidates of
// the earlier chunks from their suffix counts and writes its own chunk's:
// wave w owns entries [2048 w, 2048 w + 2048) of the chunk, read in two
// rounds of one 16-byte load per lane (lane l: 16 l .. 16 l + 15 of the
// round's 1024); per-lane packed counts (above s* | at s* << 16) and a wave
// prefix sum place every lane's candidates.
__device__ __forceinline__ uint32_t vote_counts(const u32x4_t& vv, int i, int n, int star) {
  uint32_t c = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int b = (int)((vv[e >> 2] >> (8 * (e & 3))) & 0xffu);
    if (i + e < n) c += b > star ? 1u : (b == star ? 0x10000u : 0u);
  }
  return c;
}

__global__ __launch_bounds__(256) void cand_write_kernel(const uint8_t* votes, int ldv, int n,
                                                         int n_chunks, int C,
                                                         const int32_t* tot_ge,
                                                         const int32_t* chunk_ge, int32_t* win,
                                                         int32_t* cand) {
  __shared__ int tg[kGe + 1];
  __shared__ int s_star;
  __shared__ int pa[4], pb[4], wt[4];
  const int h = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int tgv = 0;
  if (tid < kGe) tgv = tot_ge[(int64_t)h * kGe + tid];
  const int i0 = chunk * kChunk + wave * (kChunk / 4);
  const uint8_t* vr = votes + (int64_t)h * ldv;
  u32x4_t vv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = i0 + r * 1024 + 16 * lane;
    vv[r] = i < n ? *(const u32x4_t*)(vr + i) : u32x4_t{0, 0, 0, 0};
  }
  if (tid < kGe) tg[tid] = tgv;
  if (tid == 0) {
    tg[kGe] = 0;
    s_star = -1;   // stays -1 only if C exceeds the entry count
    if (h == 0 && chunk == 0) {
      win[0] = 0;
      win[1] = C;
    }
  }
  lds_barrier();
  if (tid < kGe && tg[tid] >= C && tg[tid + 1] < C) s_star = tid;
  lds_barrier();
  const int star = s_star;
  const int need = star < 0 ? 0 : C - tg[star + 1];
  // candidates above / at s* in the earlier chunks and at s* in this one
  const int32_t* cg = chunk_ge + (int64_t)h * n_chunks * kGe;
  int pg = 0, pe = 0;
  for (int c2 = tid; c2 < chunk; c2 += 256) {
    const int gt = cg[(int64_t)c2 * kGe + star + 1];
    pg += gt;
    if (star >= 0) pe += cg[(int64_t)c2 * kGe + star] - gt;
  }
  const int eq_own = star < 0 ? 0
                              : cg[(int64_t)chunk * kGe + star] - cg[(int64_t)chunk * kGe + star + 1];
  const int sg = wave_total(wave_incl_scan(pg)), se = wave_total(wave_incl_scan(pe));
  // this wave's counts, both rounds
  uint32_t cnt[2];
  int incl[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    cnt[r] = vote_counts(vv[r], i0 + r * 1024 + 16 * lane, n, star);
    incl[r] = wave_incl_scan((int)cnt[r]);
  }
  const int r0_tot = wave_total(incl[0]);
  if (lane == 0) {
    pa[wave] = sg;
    pb[wave] = se;
    wt[wave] = r0_tot + wave_total(incl[1]);
  }
  lds_barrier();
  int gt_before = 0, eq_before = 0, ow = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    gt_before += pa[v];
    eq_before += pb[v];
    if (v < wave) ow += wt[v];
  }
  const int off = gt_before + min(eq_before, need);
  const int take = max(0, min(eq_own, need - eq_before));
  int32_t* crow = cand + (int64_t)h * C;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int before = ow + (incl[r] - (int)cnt[r]) + (r ? r0_tot : 0);
    int ab = before & 0xffff, eb = before >> 16;
    if ((cnt[r] & 0xffffu) || ((cnt[r] >> 16) && eb < take)) {
      const int i = i0 + r * 1024 + 16 * lane;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int b = i + e < n ? (int)((vv[r][e >> 2] >> (8 * (e & 3))) & 0xffu) : -1;
        if (b < 0) {
        } else if (b > star) {
          const int d = off + ab + min(eb, take);
          if (d < C) crow[d] = i + e;
          ++ab;
        } else if (b == star) {
          if (eb < take && off + ab + eb < C) crow[off + ab + eb] = i + e;
          ++eb;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ rerank --
// est_i = max_g fl(|q_g| * tree16_b fl(w_ib * tree8_j fl(v_ibj * q~_gbj))).
// Grid (ceil(C / 256), H), 256 threads: a 16-lane group takes 16 consecutive
// candidates, lane b holding subspace b of each (its codes word and weight,
// one non-temporal 8-byte load: a candidate's 16 lanes read one 128-byte line; with codes
// and weights in separate arrays each candidate cost two lines and the
// kernel 14.6 us at C = 20,962 x 8 heads).  A nibble's signed level
// comes from a 16-entry LDS table (one lookup instead of a compare/select
// chain).  The tree16 over the subspaces is a butterfly in which every level
// halves the candidates a lane carries (lanes b, b ^ m add the same operands
// as the tree's level m), so a group's 16 sums take 15 lane exchanges per
// query head and lane u ends with candidate u's.  The first workgroup of a
// head also zeroes the head's vote totals for the next call.
template <int G>
__global__ __launch_bounds__(256) void rerank_kernel(const uint32_t* cw, int cap,
                                                     int n, const int32_t* cand, int C,
                                                     const float* qt, const float* qn,
                                                     CodebookArgs cb, float* est,
                                                     int32_t* tot_ge) {
  __shared__ float vtab[16];
  const int h = blockIdx.y, tid = threadIdx.x, j = tid & 15;
  const int base = (tid & 63) & ~15;   // first lane of the group
  if (blockIdx.x == 0 && tid < kGe) tot_ge[(int64_t)h * kGe + tid] = 0;   // zero for the next call
  if (tid < 16) {
    float lv = cb.levels[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if ((tid & 7) == i) lv = cb.levels[i];
    vtab[tid] = (tid & 8) ? -lv : lv;
  }
  const int ci = blockIdx.x * 256 + tid;   // lane j's own candidate (u = j)
  const int mine = min(max(cand[(int64_t)h * C + min(ci, C - 1)], 0), n - 1);
  float qv[G][8], qs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int hq = h * G + g;
    const float4 a = *(const float4*)(qt + (int64_t)hq * kD + 8 * j);
    const float4 b = *(const float4*)(qt + (int64_t)hq * kD + 8 * j + 4);
    qv[g][0] = a.x; qv[g][1] = a.y; qv[g][2] = a.z; qv[g][3] = a.w;
    qv[g][4] = b.x; qv[g][5] = b.y; qv[g][6] = b.z; qv[g][7] = b.w;
    qs[g] = qn[hq];
  }
  uint32_t code[16];
  float wb[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t ent = (int64_t)h * cap + __shfl(mine, base + u, 64);
    const uint64_t pr = __builtin_nontemporal_load((const uint64_t*)cw + ent * kSub + j);
    code[u] = (uint32_t)pr;
    wb[u] = __uint_as_float((uint32_t)(pr >> 32));
  }
  lds_barrier();   // vtab
  float x[G][16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = vtab[(code[u] >> (4 * e)) & 0xfu];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = v[e] * qv[g][e];
      x[g][u] = wb[u] * tree8(pr);
    }
  }
  float best = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int m = 8, nn = 16; m >= 1; m >>= 1, nn >>= 1) {
      const bool up = (j & m) != 0;
#pragma unroll
      for (int i = 0; i < nn / 2; ++i) {
        const float keep = up ? x[g][nn / 2 + i] : x[g][i];
        const float give = up ? x[g][i] : x[g][nn / 2 + i];
        x[g][i] = keep + xor16(give, m);
      }
    }
    const float e_g = qs[g] * x[g][0];
    best = g == 0 ? e_g : fmaxf(best, e_g);
  }
  if (ci < C) est[(int64_t)h * C + ci] = best;
}

template <int G>
void launch_rerank(const skv_index* ix, int n, const int32_t* cand, int C, const float* qt,
                   const float* qn, const CodebookArgs& ca, float* est, int32_t* tot_ge,
                   hipStream_t st) {
  rerank_kernel<G><<<dim3((C + 255) / 256, ix->H), 256, 0, st>>>(
      ix->cw, ix->cap, n, cand, C, qt, qn, ca, est, tot_ge);
}

// An empty index retrieves nothing.
__global__ void empty_kernel(int k_final, int32_t* idx, int32_t* n_cand) {
  const int h = blockIdx.x;
  for (int i = threadIdx.x; i < k_final; i += blockDim.x) idx[(int64_t)h * k_final + i] = -1;
  if (threadIdx.x == 0) n_cand[h] = 0;
}

// workspace of a retrieval; the zero-kept part of the top-k workspace and
// the vote totals are zero when a call starts and are left zero
struct RetrieveWs {
  int32_t* tot_ge;    // [H][98]: #(S >= v) over all entries (kept zero)
  void* topk;         // top-k workspace (its first region is kept zero)
  uint32_t* lut;      // [H][16][256] packed tier weights of the G query heads
  float* qt;          // [Hq][128]
  float* qn;          // [Hq]
  uint8_t* votes;     // [H][ldv], ldv = n rounded up to 16
  int32_t* chunk_ge;  // [H][n_chunks][98]: #(S >= v) per chunk
  int32_t* win;       // [2]: top-k window over the candidates
  int32_t* cand;      // [H][C]
  float* est;         // [H][C]

  static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t layout(RetrieveWs* w, char* base, int H, int G, int n, int C) {
    const int n_chunks = (n + kChunk - 1) / kChunk;
    const int Hq = H * G;
    size_t o = 0;
    auto take = [&](size_t bytes) {
      char* p = base ? base + o : nullptr;
      o += al(bytes);
      return p;
    };
    // the regions kept zero between calls (the vote totals, then the top-k
    // workspace's own) come first, at offsets that do not depend on n or C,
    // so one workspace serves an index that grows between calls
    int32_t* tot = (int32_t*)take((size_t)H * kGe * 4);
    void* tk = take(topk_workspace_bytes(H, std::max(C, 1)));
    uint32_t* lut = (uint32_t*)take((size_t)H * kSub * kCent * 4);
    float* qt = (float*)take((size_t)Hq * kD * 4);
    float* qn = (float*)take((size_t)Hq * 4);
    uint8_t* votes = (uint8_t*)take((size_t)H * ((n + 15) & ~15));
    int32_t* cge = (int32_t*)take((size_t)H * n_chunks * kGe * 4);
    int32_t* win = (int32_t*)take(8);
    int32_t* cand = (int32_t*)take((size_t)H * C * 4);
    float* est = (float*)take((size_t)H * C * 4);
    if (w) {
      w->topk = tk;
      w->tot_ge = tot;
      w->lut = lut;
      w->qt = qt;
      w->qn = qn;
      w->votes = votes;
      w->chunk_ge = cge;
      w->win = win;
      w->cand = cand;
      w->est = est;
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
  return ix && ix->ids && ix->cw && ix->hist && ix->pos && ix->H >= 1 &&
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
  // about 512 workgroups or more: 16 keys each for an Update Buffer flush,
  // up to 2048 for a prefill
  const int64_t want = ((int64_t)n_keys * kv->H + 511) / 512;
  const int per_wg = (int)std::min<int64_t>(kEncPerWG, std::max<int64_t>(16, (want + 15) / 16 * 16));
  dim3 grid((n_keys + per_wg - 1) / per_wg, kv->H);
  encode_kernel<<<grid, 256, 0, stream>>>(a, b, t0, n_keys, index->n, index->cap, per_wg,
                                          cb->signs, cb_args(cb), index->ids, index->cw,
                                          index->hist, index->pos);
  if (hipGetLastError() != hipSuccess) return SKV_ELAUNCH;
  index->n += n_keys;
  return SKV_OK;
}

skv_status sparsekv_update_buffer(const skv_codebook* cb, const skv_kv* kv, int32_t b,
                                  int32_t seq_len, int32_t sink, int32_t local, int32_t update,
                                  skv_index* index, int32_t* flushed, hipStream_t stream) {
  if (!kv || !index) return SKV_EINVAL;
  if (sink < 0 || local < 0 || update < 1 || seq_len < 0 || seq_len > kv->L_max) return SKV_EINVAL;
  const int64_t end = (int64_t)sink + index->n;   // retrieval region [sink, end)
  if (seq_len < end) return SKV_EINVAL;
  // whole buffers of `update` tokens that are full move into Local; as many
  // of the oldest Local tokens move on into the index
  const int64_t tail = seq_len - end;
  const int64_t n_buf = tail >= (int64_t)local + update ? (tail - local) / update : 0;
  if (flushed) *flushed = (int32_t)n_buf;
  if (n_buf == 0) return SKV_OK;
  return sparsekv_encode(cb, kv, b, (int32_t)end, (int32_t)(end + n_buf * update), index, stream);
}

size_t sparsekv_retrieve_workspace_size(const skv_index* index, int32_t G, double beta,
                                        int32_t k_final) {
  if (!index || index->H < 1 || index->n < 0 || G < 1 || k_final < 1 || !(beta > 0)) return 0;
  const int C = n_candidates(index->n, beta);
  return RetrieveWs::layout(nullptr, nullptr, index->H, G, index->n, std::max(C, 1));
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
  RetrieveWs::layout(&w, (char*)ws, H, G, n, C);
  const int ldv = (n + 15) & ~15;
  int32_t* cand = (trace && trace->cand) ? trace->cand : w.cand;
  float* est = (trace && trace->est) ? trace->est : w.est;
  const int n_chunks = (n + kChunk - 1) / kChunk;

  TierArgs ta;
  ta.t_rho = (int)ceil(rho * (double)n);
  const double fr[6] = {0.05, 0.15, 0.30, 0.50, 0.75, 1.0};
  for (int i = 0; i < 6; ++i) ta.T[i] = (int)ceil(fr[i] * (double)ta.t_rho);
  const CodebookArgs ca = cb_args(cb);

  query_lut_kernel<<<dim3(kSub, H, 4), 256, 0, stream>>>((const uint16_t*)q, G, cb->signs, ca.c,
                                                         index->hist, ta, w.qt, w.qn,
                                                         (uint8_t*)w.lut);
  vote_kernel<<<dim3(n_chunks, H), 256, 0, stream>>>(index->ids, index->cap, n, w.lut, w.votes,
                                                     ldv, trace ? trace->votes : nullptr,
                                                     w.chunk_ge, n_chunks, w.tot_ge);
  cand_write_kernel<<<dim3(n_chunks, H), 256, 0, stream>>>(w.votes, ldv, n, n_chunks, C, w.tot_ge,
                                                           w.chunk_ge, w.win, cand);
  switch (G) {
    case 1: launch_rerank<1>(index, n, cand, C, w.qt, w.qn, ca, est, w.tot_ge, stream); break;
    case 2: launch_rerank<2>(index, n, cand, C, w.qt, w.qn, ca, est, w.tot_ge, stream); break;
    case 3: launch_rerank<3>(index, n, cand, C, w.qt, w.qn, ca, est, w.tot_ge, stream); break;
    default: launch_rerank<4>(index, n, cand, C, w.qt, w.qn, ca, est, w.tot_ge, stream); break;
  }
  hipError_t e = launch_topk(est, H, H, C, w.win, w.win + 1, k_final, idx, n_cand, w.topk, false,
                             stream, cand, index->pos, C);
  if (e != hipSuccess) return SKV_ELAUNCH;
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // extern "C"
