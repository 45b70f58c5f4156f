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
// wave) owns one split of the position list, at most 128 rows at a time:
// threads resolve the rows' addresses together, then the load unit copies
// the rows global -> LDS itself (global_load_lds_dwordx4, no registers
// involved), so a block costs one chain of table load, copy and wait.  Per
// 32-token chunk
//   S^T[16 tokens x 16 heads] = K_half . Q^T     2 x 18 v_mfma_f32_16x16x32_bf16
// leaves each lane P[head][8 tokens] (4 of each half), which is the A operand
// of the value product with k slot 8 g4 + e <-> token 4 g4 + e (e < 4) or
// 16 + 4 g4 + e - 4, and
//   O[16 heads x 512] += P . V                    32 x v_mfma_f32_16x16x32_bf16
// with P split into a bf16 head and a bf16 tail (two products), which keeps
// the probabilities to ~16 significant bits.  The value operand (8 tokens x
// 1 dim per lane, same k mapping) is read straight from the token-major rows
// with two transposing LDS reads ds_read_b64_tr_b16: within 16 lanes, lane j
// receives element j % 4 of the 8-byte pieces addressed by lanes j / 4 + 4 i,
// so lane (p, g4) addresses token 4 g4 + p / 4 of a half, dims
// 16 c + 4 (p % 4).  An online softmax (log2 domain) runs across chunks; the
// split partials are merged exactly by log-sum-exp.
#include <algorithm>

#include "skv_device.h"
#include "skv_listsel.h"

namespace skv {

namespace {

constexpr int kDk = 576, kDv = 512;
constexpr int kRowPad = kDk + 8;        // LDS row stride (bf16 elements; 1168 B, 16-byte aligned)
constexpr int kBlock = 128;             // latent rows resident in LDS at a time
constexpr int kNC = kDk / 32;           // 18 MFMA k-steps for the logits
constexpr int kVB = kDv / 16;           // 32 value column blocks

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Copy one 1152-byte latent row into LDS with the load unit: lanes 0..63
// move bytes 0..1023, lanes 0..7 the last 128.
__device__ __forceinline__ void row_to_lds(const uint16_t* src, uint16_t* dst, int lane) {
  __builtin_amdgcn_global_load_lds((gbl_void_t)(src + 8 * lane), (lds_void_t)dst, 16, 0, 0);
  if (lane < 8)
    __builtin_amdgcn_global_load_lds((gbl_void_t)(src + 512 + 8 * lane), (lds_void_t)(dst + 512),
                                     16, 0, 0);
}

// S^T of one 32-token chunk for 16 heads: S[hf] (lane (n, g4): tokens
// 16 hf + 4 g4 + i of the chunk, head n) = sum over the 18 k-steps j of
// K_hf[16 x 32] . Q^T[32 x 16], K_hf from the token-major LDS rows (krow:
// this lane's piece of token n, k-step 0) and the B operand qf(j).  The
// LDS reads go in batches of 6 k-steps, all issued before their products:
// one k-step at a time, each product waited for its own reads (1.9 us per
// chunk for the 36 products).
template <class QF>
__device__ __forceinline__ void logits_from_lds(const uint16_t* krow, QF&& qf, f32x4_t (&S)[2]) {
  constexpr int kBatch = 6;
  static_assert(kNC % kBatch == 0, "k-step batches");
  S[0] = S[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j0 = 0; j0 < kNC; j0 += kBatch) {
    bf16x8_t k0[kBatch], k1[kBatch], qb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u;
      k0[u] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(krow + 32 * j));
      k1[u] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(krow + 16 * kRowPad + 32 * j));
      qb[u] = qf(j);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[u], qb[u], S[0], 0, 0, 0);
      S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[u], qb[u], S[1], 0, 0, 0);
    }
  }
}

// 4 tokens x 1 dim of the value operand from token-major LDS rows
__device__ __forceinline__ u32x2_t value_tr(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mla_split_kernel(
    KvArgs kv, const uint16_t* q, int G, const int32_t* idx, int k, const int32_t* lo_p,
    const int32_t* hi_p, float scale_log2, int n_split, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t rows[kBlock * kRowPad];
  __shared__ int64_t roff[kBlock];
  // grid (n_split, H x head groups, B): a workgroup serves WAVES x 16 of the
  // G query heads; the head groups of a split sit 8-aligned apart in the
  // dispatch order (n_split is a multiple of 8), so they share an XCD and its
  // L2 copy of the split's latent rows
  const int n_hg = G / (16 * WAVES);
  const int s = blockIdx.x, h = blockIdx.y / n_hg, hg = blockIdx.y - h * n_hg, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int head0 = (hg * WAVES + wave) * 16;     // this wave's first query head

  const int seq = min(kv.seq_len[b], kv.L_max);
  const int lo = max(0, min(lo_p[b], seq));
  const int hi = max(lo, min(hi_p[b], seq));
  const int n_list = k + lo + (seq - hi);
  const int chunk = (n_list + n_split - 1) / n_split;
  const int p0 = s * chunk, p1 = min(n_list, p0 + chunk);
  const int32_t* irow = idx + ((int64_t)b * kv.H + h) * k;
  const uint16_t* kb = (const uint16_t*)kv.k;
  const uint16_t* qhead = q + ((int64_t)b * kv.H + h) * G * kDk;   // a finite stand-in row

  // Q^T operand: lane (n, g4), step j holds q[head0 + n][8 (4j + g4) .. +8]
  bf16x8_t Qf[kNC];
  const uint16_t* qrow = qhead + (int64_t)(head0 + n) * kDk;
#pragma unroll
  for (int j = 0; j < kNC; ++j)
    Qf[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qrow + 8 * (4 * j + g4)));

  // online softmax state for head head0 + n (replicated over g4)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t O[kVB];
#pragma unroll
  for (int c = 0; c < kVB; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int q0 = p0; q0 < p1; q0 += kBlock) {
    const int cnt = min(kBlock, p1 - q0);
    const int n_rows = (cnt + 31) & ~31;          // rows staged: whole 32-token chunks
    // element offset of each latent row, or -1 (dead, or past the split)
    for (int r = tid; r < kBlock; r += WAVES * 64) {
      int64_t ro = -1;
      if (r < cnt) {
        const int pos = q0 + r;
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
      roff[r] = ro;
    }
    __syncthreads();   // also: every wave is done with the previous block's rows
    // wave w copies rows w, w + WAVES, ...; dead rows get the query row
    // instead (finite; their weight is zero)
    for (int r = wave; r < n_rows; r += WAVES) {
      const int64_t ro = roff[r];
      row_to_lds(ro >= 0 ? kb + ro : qhead, rows + r * kRowPad, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int c0 = 0; c0 < cnt; c0 += 32) {
      // S^T[token 16 hf + 4 g4 + i][head n] for the two 16-token halves
      f32x4_t S[2];
      logits_from_lds(rows + (c0 + n) * kRowPad + 8 * g4, [&](int j) { return Qf[j]; }, S);
      float z[8];
      float cm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tk = c0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
        const bool ok = tk < cnt && roff[tk] >= 0;
        z[e] = ok ? S[e >> 2][e & 3] * scale_log2 : -INFINITY;
        cm = fmaxf(cm, z[e]);
      }
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float m_new = fmaxf(m_run, cm);
      float p[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = m_new == -INFINITY ? 0.f : exp2f(z[e] - m_new);
        ps += p[e];
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
      // P as the A operand (head n, k slots 8 g4 .. +7), split into head + tail
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t h0 = f32_to_bf16_rne(p[e]), h1 = f32_to_bf16_rne(p[e + 1]);
        const uint32_t l0 = f32_to_bf16_rne(p[e] - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(p[e + 1] - __uint_as_float(h1 << 16));
        ph[e >> 1] = h0 | (h1 << 16);
        pl[e >> 1] = l0 | (l1 << 16);
      }
      const bf16x8_t Ph = __builtin_bit_cast(bf16x8_t, u32x4_t{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8_t Pl = __builtin_bit_cast(bf16x8_t, u32x4_t{pl[0], pl[1], pl[2], pl[3]});
      // value operand: lane (n, g4) addresses token 16 hf + 4 g4 + n / 4, dims 4 (n % 4) .. + 3
      const uint16_t* v0 = rows + (c0 + 4 * g4 + (n >> 2)) * kRowPad + 4 * (n & 3);
      const uint16_t* v1 = v0 + 16 * kRowPad;
#pragma unroll
      for (int c = 0; c < kVB; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[c][i] *= oc[i];
        const u32x2_t a = value_tr(v0 + 16 * c), bb = value_tr(v1 + 16 * c);
        const bf16x8_t Vf = __builtin_bit_cast(bf16x8_t, u32x4_t{a[0], a[1], bb[0], bb[1]});
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ph, Vf, O[c], 0, 0, 0);
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pl, Vf, O[c], 0, 0, 0);
      }
    }
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

// splits: a multiple of 8 (see the head-group placement), ~64 rows each
int mla_splits(int k) { return std::max(8, std::min(64, (k + 63) / 64 + 7) / 8 * 8); }

// ------------------------------------------ selection fused with attention --
// After the slice listing of a long row (the exact top-k's list in the top-k
// workspace) or a scan that listed segment candidates (SEG), one kernel
// finishes the selection and attends: grid (n_split, rows x head parts), 1024
// threads.  Every workgroup of a row resolves the row's exact selection by
// itself (list_select or seg_select; the row alone when those do not settle
// it), so no workgroup waits for another; split s takes the selected keys of
// ranks [s n_sel / n_split, (s + 1) n_sel / n_split) and an equal share of
// the always-attended tokens (t < lo, t >= hi), stages their latent rows in
// LDS 64 at a time with the load unit, and attends for its 16 (kRowWaves /
// DP) query heads, whose rows it also stages in LDS.  The 16 waves are
// 16-head groups x DP parts of the value dims.  Per staged block (up to two
// 32-token chunks) waves 0 and 1 of a head group form the logits of one chunk
// each at the same time (2 x 18 v_mfma_f32_16x16x32_bf16), exchange their
// maxima through LDS (one barrier), update the online softmax with the
// block's max and leave the probability fragments (bf16 head + tail, the A
// operand of the value product) and the rescale factor in LDS; after a second
// barrier every wave of the group applies them to its 32 / DP column blocks
// of 16 value dims for both chunks (one chunk's logits after another took
// 1.56 us each).  Per-wave state stays small (the accumulators of 512 / DP
// dims), which 1024-thread workgroups need.  Split 0 of head part 0 writes
// idx and count.  The rows' histograms and list counters are zeroed by the
// merge kernel that follows.
constexpr int kFuseRows = 64;          // latent rows staged at a time
constexpr int kFuseSlices = 1024;      // listing slices of a row this kernel reads

template <int DP, bool SEG>
__global__ __launch_bounds__(kRowThreads) void mla_list_kernel(
    KvArgs kv, const uint16_t* q, int G, const float* scores, const int32_t* lo_p,
    const int32_t* hi_p, int k, TopkWs ws, int n_slices, float scale_log2, int n_split,
    int32_t* idx, int32_t* count, float* part, int n_seg) {
  constexpr int VB = kVB / DP;                      // value column blocks per wave
  constexpr int NHG = kRowWaves / DP;               // 16-head groups per workgroup
  constexpr int kHeadsPerWg = 16 * NHG;
  __shared__ RowSelLds L;
  __shared__ int s_off[kFuseSlices + 1], s_at[kFuseSlices];
  __shared__ int klist_n;
  __shared__ __attribute__((aligned(16))) uint16_t rows[kFuseRows * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t qs[kHeadsPerWg * kRowPad];
  __shared__ u32x4_t pfrag[NHG][2][64][2];          // [group][chunk][lane][head, tail]
  __shared__ float cfac[NHG][16];                   // rescale factor per head
  __shared__ float cmax[NHG][2][16];                // the chunks' logit maxima per head
  __shared__ float lsum[NHG][16];                   // the second logit wave's weight sums
  __shared__ int64_t roff[kFuseRows];
  const int n_hp = (G + kHeadsPerWg - 1) / kHeadsPerWg;   // head parts per row
  const int s = blockIdx.x, row = blockIdx.y / n_hp, hp = blockIdx.y - row * n_hp;
  const int b = row / kv.H, h = row - b * kv.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = row_wave();
  const int n = lane & 15, g4 = lane >> 4;
  const int hg = wave / DP, dp = wave - hg * DP;
  const int head0 = hp * kHeadsPerWg + hg * 16;
  const bool on = head0 < G;                        // a group past the heads only helps stage
  const uint16_t* qhead = q + ((int64_t)b * kv.H + h) * G * kDk;   // a finite stand-in row

  // this workgroup's query rows, staged by the load unit while the selection
  // runs (finite stand-ins past G; no registers involved)
  for (int r = wave; r < kHeadsPerWg; r += kRowWaves) {
    const int hd = hp * kHeadsPerWg + r;
    row_to_lds(qhead + (int64_t)(hd < G ? hd : 0) * kDk, qs + r * kRowPad, lane);
  }
  // the sequence's block table too, into the latent-row area (free until the
  // first block of rows is staged), so the first block's addresses need no
  // table load after the selection (1.6 us of dependent loads otherwise)
  const int n_bt = kv.block_table && !kv.token_table ? (kv.L_max >> 4) : 0;
  const bool bt_lds = n_bt > 0 && n_bt % 256 == 0 && n_bt * 4 <= (int)sizeof(rows) &&
                      ((uintptr_t)kv.block_table & 15) == 0;
  const int32_t* btl = (const int32_t*)rows;
  if (bt_lds) {
    const int32_t* src = kv.block_table + (int64_t)b * n_bt;
    for (int c = wave; c < n_bt / 256; c += kRowWaves)
      __builtin_amdgcn_global_load_lds((gbl_void_t)(src + c * 256 + 4 * lane),
                                       (lds_void_t)(rows + c * 512), 16, 0, 0);
  }

  // 1. the row's exact selection, positions ascending in L.hist[0 .. n_sel)
  // (from the scan's segment candidates with SEG, else from the slice
  // listing's list; the row alone when those do not settle it)
  auto keep = [&](int dst, int p, uint32_t) { L.hist[dst] = (uint32_t)p; };
  const uint4 gv = SEG ? make_uint4(0u, 0u, 0u, 0u) : hist_bins_summed(ws, row);
  int n_sel = -1;
  if constexpr (SEG)
    n_sel = seg_select(ws, row, n_seg, k, L, keep);
  else if (ws.meta[2 * row + 1] >= 0)
    n_sel = list_select(ws, row, k, n_slices, gv, L, s_off, s_at, keep);
  if (n_sel < 0) {
    lds_barrier();   // every thread is past its reads of L
    if constexpr (SEG)
      n_sel = fallback_select_nohist(scores, row, kv.H, kv.L_max, lo_p, hi_p, k, L, klist_n);
    else
      n_sel = fallback_select(scores, row, kv.H, kv.L_max, lo_p, hi_p, k,
                              ws.hist + (int64_t)row * ws.copies * kBins, L, klist_n, gv);
  } else {
    lds_barrier();
  }
  if (s == 0 && hp == 0) {
    int32_t* orow = idx + (int64_t)row * k;
    for (int i = tid; i < k; i += kRowThreads) orow[i] = i < n_sel ? (int)L.hist[i] : -1;
    if (tid == 0) count[row] = n_sel;
  }
  // 2. this split's share: selected ranks [r0, r1), always-attended [x0, x1)
  const int seq = min(kv.seq_len[b], kv.L_max);
  const int lo = max(0, min(lo_p[b], seq));
  const int hi = max(lo, min(hi_p[b], seq));
  const int n_extra = lo + (seq - hi);
  const int r0 = (int)((int64_t)n_sel * s / n_split), r1 = (int)((int64_t)n_sel * (s + 1) / n_split);
  const int x0 = (int)((int64_t)n_extra * s / n_split);
  const int x1 = (int)((int64_t)n_extra * (s + 1) / n_split);
  const int n_list = r1 - r0, n_att = n_list + (x1 - x0);
  const uint16_t* kb = (const uint16_t*)kv.k;

  // online softmax state of head head0 + n, kept by the group's two logit
  // waves (dp 0 and 1: the two 32-token chunks of a staged block); both
  // track the same running max, each the sum of its own chunks' weights
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t O[VB];
#pragma unroll
  for (int c = 0; c < VB; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* qrow = qs + (hg * 16 + n) * kRowPad;
  const bool logit_wave = on && dp < 2;
  if (bt_lds) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // the block table is in LDS

  for (int q0 = 0; q0 < n_att; q0 += kFuseRows) {
    const int cnt = min(kFuseRows, n_att - q0);
    const int n_rows = (cnt + 31) & ~31;
    const int nch = n_rows >> 5;   // 32-token chunks of this block (1 or 2)
    if (tid < kFuseRows) {
      int64_t ro = -1;
      if (tid < cnt) {
        const int i = q0 + tid;
        int t;
        if (i < n_list) {
          t = (int)L.hist[r0 + i];
        } else {
          const int x = x0 + (i - n_list);
          t = x < lo ? x : hi + (x - lo);
        }
        int64_t slot;
        if (bt_lds && q0 == 0)   // slot_of with the table entry from LDS (seq <= L_max)
          slot = (t < 0 || t >= seq) ? -1 : (int64_t)btl[t >> 4] * 16 + (t & 15);
        else
          slot = slot_of(kv, b, t);
        ro = slot >= 0 ? row_elem(kv, b, h, slot, kDk) : -1;
      }
      roff[tid] = ro;
    }
    __syncthreads();   // also: every wave is done with the previous block's rows
    for (int r = wave; r < n_rows; r += kRowWaves) {
      const int64_t ro = roff[r];
      row_to_lds(ro >= 0 ? kb + ro : qhead, rows + r * kRowPad, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // the staged latent rows (and, the first time, the query rows)
    // logits of chunk dp by the group's waves dp < 2, both chunks at once:
    // S^T[token 16 hf + 4 g4 + i][head n] for the chunk's two 16-token halves
    float z[8];
    float cm = -INFINITY;
    if (logit_wave && dp < nch) {
      const int c0 = 32 * dp;
      f32x4_t S[2];
      const uint16_t* qg = qrow + 8 * g4;
      logits_from_lds(rows + (c0 + n) * kRowPad + 8 * g4, [&](int j) {
        return __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qg + 32 * j));
      }, S);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tk = c0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
        const bool ok = tk < cnt && roff[tk] >= 0;
        z[e] = ok ? S[e >> 2][e & 3] * scale_log2 : -INFINITY;
        cm = fmaxf(cm, z[e]);
      }
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = -INFINITY;
    }
    if (logit_wave && g4 == 0) cmax[hg][dp][n] = cm;
    lds_barrier();   // the two chunks' maxima
    if (logit_wave) {
      const float m_new = fmaxf(m_run, fmaxf(cmax[hg][0][n], cmax[hg][1][n]));
      float p[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = m_new == -INFINITY ? 0.f : exp2f(z[e] - m_new);
        ps += p[e];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      const float corr = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run = l_run * corr + ps;
      m_run = m_new;
      if (dp < nch) {
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t h0 = f32_to_bf16_rne(p[e]), h1 = f32_to_bf16_rne(p[e + 1]);
          const uint32_t l0 = f32_to_bf16_rne(p[e] - __uint_as_float(h0 << 16));
          const uint32_t l1 = f32_to_bf16_rne(p[e + 1] - __uint_as_float(h1 << 16));
          ph[e >> 1] = h0 | (h1 << 16);
          pl[e >> 1] = l0 | (l1 << 16);
        }
        pfrag[hg][dp][lane][0] = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
        pfrag[hg][dp][lane][1] = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
      }
      if (dp == 0 && g4 == 0) cfac[hg][n] = corr;
    }
    lds_barrier();   // the group's probabilities of both chunks and the rescale factor
    if (on) {
      float oc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) oc[i] = cfac[hg][4 * g4 + i];
#pragma unroll
      for (int c = 0; c < VB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[c][i] *= oc[i];
      for (int ch = 0; ch < nch; ++ch) {
        const bf16x8_t Ph = __builtin_bit_cast(bf16x8_t, pfrag[hg][ch][lane][0]);
        const bf16x8_t Pl = __builtin_bit_cast(bf16x8_t, pfrag[hg][ch][lane][1]);
        const uint16_t* v0 =
            rows + (32 * ch + 4 * g4 + (n >> 2)) * kRowPad + 4 * (n & 3) + 16 * VB * dp;
        const uint16_t* v1 = v0 + 16 * kRowPad;
#pragma unroll
        for (int c = 0; c < VB; ++c) {
          const u32x2_t a = value_tr(v0 + 16 * c), bb = value_tr(v1 + 16 * c);
          const bf16x8_t Vf = __builtin_bit_cast(bf16x8_t, u32x4_t{a[0], a[1], bb[0], bb[1]});
          O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ph, Vf, O[c], 0, 0, 0);
          O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pl, Vf, O[c], 0, 0, 0);
        }
      }
    }
  }
  // the second logit wave's weight sum joins the first's
  if (logit_wave && dp == 1 && g4 == 0) lsum[hg][n] = l_run;
  lds_barrier();
  if (logit_wave && dp == 0) l_run += lsum[hg][n];

  // 3. the split partial: O[head][512], max, sum (lane holds heads 4 g4 + i);
  // an empty share never waited for the staged query rows
  __builtin_amdgcn_s_waitcnt(0);
  if (!on) return;
  const int stride = kDv + 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = head0 + 4 * g4 + i;
    float* dst = part + (((int64_t)row * G + hd) * n_split + s) * stride + 16 * VB * dp;
#pragma unroll
    for (int c = 0; c < VB; ++c) dst[16 * c + n] = O[c][i];
  }
  if (dp == 0 && g4 == 0) {
    float* dst = part + (((int64_t)row * G + head0 + n) * n_split + s) * stride;
    dst[kDv] = m_run;
    dst[kDv + 1] = l_run;
  }
}

constexpr int kFuseSplits = 32;        // splits of the fused selection + attention

}  // namespace

bool mla_supported(const KvArgs& kv, int G) {
  return kv.bf16 && kv.v == nullptr && kv.d_k == kDk && kv.d_v == kDv &&
         (G == 16 || G == 32 || G == 64 || G == 128);
}

size_t mla_workspace_bytes(const KvArgs& kv, int G, int k) {
  return (size_t)kv.B * kv.H * G * mla_splits(k) * (kDv + 2) * sizeof(float);
}

// The exact top-k of long rows (more than one 32768-slot sweep) finished
// from the slice listing inside the attention kernel: G in {16, 32, 64, 128},
// k <= 4096, at most kFuseSlices listing slices per row.
bool mla_list_supported(const KvArgs& kv, int G, int k) {
  return mla_supported(kv, G) && k >= 1 && k <= kBins && row_slots_max(kv.L_max) > kSweep &&
         topk_slices(kv.L_max) <= kFuseSlices;
}

size_t mla_list_partial_bytes(const KvArgs& kv, int G) {
  return (size_t)kv.B * kv.H * G * kFuseSplits * (kDv + 2) * sizeof(float);
}

size_t mla_select_attend_partial_bytes(const KvArgs& kv, int G, int k) {
  return std::max(mla_list_partial_bytes(kv, G), mla_workspace_bytes(kv, G, k));
}

hipError_t launch_mla_list_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                  const int32_t* lo, const int32_t* hi, int k, void* topk_ws,
                                  float scale, int32_t* idx, int32_t* count, float* part,
                                  float* out, hipStream_t st, int n_seg) {
  const int rows = kv.B * kv.H;
  const TopkWs ws = TopkWs::carve(topk_ws, rows, kv.L_max);
  const int ns = topk_listing_slices(rows, kv.L_max);
  if (ns > kFuseSlices) return hipErrorInvalidValue;
  if (n_seg > kSegMax || (n_seg > 0 && k > kSegMaxK)) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (n_seg <= 0) {
    e = launch_topk_listing(scores, rows, kv.H, kv.L_max, lo, hi, k, topk_ws, st);
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const uint16_t* qq = (const uint16_t*)q;
  // 32 heads per workgroup (2 head groups x 8 dim parts); 16 heads take 16
  const int dp = G >= 32 ? 8 : 16;
  const int n_hp = (G + 16 * (kRowWaves / dp) - 1) / (16 * (kRowWaves / dp));
  const dim3 grid(kFuseSplits, rows * n_hp);
#define SKV_MLA_LIST(D, SG)                                                                     \
  mla_list_kernel<D, SG><<<grid, kRowThreads, 0, st>>>(kv, qq, G, scores, lo, hi, k, ws, ns,     \
                                                       scale_log2, kFuseSplits, idx, count, part, \
                                                       n_seg)
  if (dp == 8) {
    if (n_seg > 0) SKV_MLA_LIST(8, true); else SKV_MLA_LIST(8, false);
  } else {
    if (n_seg > 0) SKV_MLA_LIST(16, true); else SKV_MLA_LIST(16, false);
  }
#undef SKV_MLA_LIST
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_seg > 0)   // nothing of the histograms or list counters was used
    return launch_attend_reduce(part, kFuseSplits, kDv, kv.H * G, kv.B, out, st, nullptr, G, 1,
                                nullptr);
  return launch_attend_reduce(part, kFuseSplits, kDv, kv.H * G, kv.B, out, st, ws.hist, G,
                              ws.copies, ws.ctr);
}

hipError_t launch_mla_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                             const int32_t* lo, const int32_t* hi, float scale, float* out,
                             void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  const int n_split = mla_splits(k);
  float* part = (float*)ws;
  const float scale_log2 = scale * 1.4426950408889634f;
  // 32 heads (2 waves) per workgroup, 16 when G = 16
  const uint16_t* qq = (const uint16_t*)q;
  if (G == 16) {
    mla_split_kernel<1><<<dim3(n_split, kv.H, kv.B), 64, 0, st>>>(kv, qq, G, idx, k, lo, hi,
                                                                  scale_log2, n_split, part);
  } else if (G == 32 || G == 64 || G == 128) {
    mla_split_kernel<2><<<dim3(n_split, kv.H * (G / 32), kv.B), 128, 0, st>>>(
        kv, qq, G, idx, k, lo, hi, scale_log2, n_split, part);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_reduce(part, n_split, kDv, kv.H * G, kv.B, out, st);
}

}  // namespace skv
