// Fused exact top-k + gather + split-k attention of one decode step, after the
// score scan has written the scores and the rows' top-12-bit key histograms.
//
// What is computed, per sequence b and KV head h (row r = b H + h):
//   idx[r]  = the k largest finite scores of t in [lo, hi), ascending t, ties
//             to the lower t (ECHO-OSDI26 wiki page, observation 5);
//   out[b][h G + g] = softmax attention of query head g over
//             {idx[r]} U {live t < lo} U {live t >= hi}
//             (ParisKV close-reading, section 一, Eqs. (1)-(3); vToken reading
//             notes, section 3.4 Eq. (2) for the slot mapping);
// exactly what sparsekv_topk_resume followed by sparsekv_gather_attend
// compute, in one kernel plus the split merge instead of three kernels.
//
// gfx950 design.  Grid kSplits x rows, 1024 threads: 256 workgroups, one
// per CU, for the 32 rows of the GQA workload; the kSplits workgroups of a
// row are placed on one XCD (workgroups go to the 8 XCDs round-robin by id),
// so the row's scores come from memory once and then from that XCD's L2.  Every workgroup of a row
// loads the whole row of scores (coalesced, into registers) and finds the
// row's threshold redundantly, so no workgroup waits for another; workgroup s
// then takes the selected keys of ranks [s k_sel / kSplits, (s + 1) k_sel /
// kSplits) -- an equal share -- writes their entries of idx and attends over
// them plus an equal share of the sink and local tokens (17 chunks of 16
// tokens at k = 2048; every wave issues the loads of its two chunks at once).  Per wave, 16 attended tokens at a time:
// logits from matrix cores as S^T[16 tokens x 16 heads] = K_chunk . Q^T
// (4 x v_mfma_f32_16x16x32_bf16), online softmax in the log2 domain, and the
// value product on the vector ALUs with every lane owning two output dims of
// every head.  The 16 waves' (max, sum, weighted values) merge through LDS
// into the workgroup's split partial; attend_reduce_kernel merges the splits
// and zeroes the rows' histograms for the next call.
#include <algorithm>

#include "skv_internal.h"
#include "skv_listsel.h"
#include "skv_rowsel.h"

namespace skv {

namespace {

constexpr int kSplits = 8;                        // selection workgroups per row
constexpr int kShareCap = kSweep / kSplits;       // selected keys per workgroup (k <= 32768)
constexpr int kD = 128;

// Attention of one workgroup over its share of a row's tokens (step 3 of
// the fused kernels) and the merge of its 16 waves into the split partial
// (step 4): the tokens are lst[0 .. n_list) (selected positions) then the
// always-attended positions x0 .. of t < a_lo and t >= a_hi, n_att in all;
// tbl: the row's block-table entries staged in LDS, or null (slots through
// kv's table).  Qf: the MFMA B operand of the G query rows.  With out !=
// nullptr (a workgroup that attends the row's whole selection) the merged
// result is written normalised to out[row][g][:] (0 for an empty row) in
// place of a split partial.  GMAX = 1 (G = 1, one query head): lrow is the
// row's scores from the scan, which for one query head are the logits q . k
// themselves, so the key rows are not read again and only the value rows are
// gathered (the scan's fp32 dot products stand in for the attention's own),
// and the key-row and matrix-core code is not compiled in; lkey (or null):
// the listed tokens' score keys, already in LDS, so only the sink / local
// tokens' scores are read from lrow.  GMAX > 1: lrow and lkey are unused.
template <int GMAX>
__device__ __forceinline__ void attend_share(const KvArgs& kv, int G, int row, int b, int h, int s,
                                             int n_split, const int32_t* lst, int n_list, int x0,
                                             int n_att, int a_lo, int a_hi, int seq,
                                             const int32_t* tbl, const bf16x8_t (&Qf)[4],
                                             float scale_log2, float* part,
                                             int64_t (&rows_sh)[kRowWaves][2][16],
                                             float (&red)[kRowWaves][4][kD + 2],
                                             float* out = nullptr, const float* lrow = nullptr,
                                             float (*zsh)[2][16] = nullptr,
                                             const uint32_t* lkey = nullptr) {
  constexpr bool kFromScores = GMAX == 1;
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int n = lane & 15, g4 = lane >> 4;

  float m_run = -INFINITY, l_run = 0.f;   // head n (lanes n < G, every g4)
  float acc[GMAX][2];                     // dims 2 lane, 2 lane + 1 of every head
#pragma unroll
  for (int g = 0; g < GMAX; ++g) acc[g][0] = acc[g][1] = 0.f;
  const uint16_t* kb = (const uint16_t*)kv.k;
  const uint16_t* vb = (const uint16_t*)kv.v;
  // chunks c and c + kRowWaves of this wave: both chunks' loads are issued
  // before either is used
  const int n_ch = (n_att + 15) >> 4;
  for (int c0 = wave; c0 < n_ch; c0 += 2 * kRowWaves) {
    if (lane < 32) {
      const int u = lane >> 4;
      const int i = (c0 + u * kRowWaves) * 16 + (lane & 15);
      int t = -1;
      if (i < n_att) {
        if (i < n_list) {
          t = lst[i];
        } else {
          const int x = x0 + (i - n_list);
          t = x < a_lo ? x : a_hi + (x - a_lo);
        }
      }
      int64_t slot = -1;
      if (t >= 0) {
        if (tbl) {
          const int e = t < seq ? tbl[t >> 4] : -1;
          slot = e < 0 ? -1 : (int64_t)e * 16 + (t & 15);
        } else {
          slot = slot_of(kv, b, t);
        }
      }
      rows_sh[wave][u][lane & 15] = slot >= 0 ? row_elem(kv, b, h, slot, kD) : -1;
      if constexpr (kFromScores)
        zsh[wave][u][lane & 15] =
            slot < 0 ? -INFINITY
                     : (lkey && i < n_list ? key_score(lkey[i]) : lrow[t]) * scale_log2;
    }
    bf16x8_t Kf[kFromScores ? 1 : 2][4];
    uint32_t Vw[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (!kFromScores) {
        const int64_t rk = rows_sh[wave][u][n];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t v = rk >= 0 ? ld16((const char*)(kb + rk + 8 * (4 * j + g4)))
                                    : u32x4_t{0, 0, 0, 0};
          Kf[u][j] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int64_t rv = rows_sh[wave][u][t];
        // one wave load per V row (its two whole lines), read once: non-temporal
        // (token-pool select + attend 68.5 -> 67.3 us)
        Vw[u][t] = rv >= 0 ? __builtin_nontemporal_load((const uint32_t*)(vb + rv + 2 * lane)) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (c0 + u * kRowWaves >= n_ch) break;
      f32x4_t S = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!kFromScores) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf[u][j], Qf[j], S, 0, 0, 0);
      }
      // lane (n, g4) holds the logits of query head n for tokens 4 g4 .. 4 g4 + 3
      float z[4], cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rows_sh[wave][u][4 * g4 + i] >= 0;
        z[i] = !ok ? -INFINITY : kFromScores ? zsh[wave][u][4 * g4 + i] : S[i] * scale_log2;
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
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
          const float cgr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), g));
          // the 16 weights of head g first (scalars read back to back), then
          // the products
          float pg[16];
#pragma unroll
          for (int t = 0; t < 16; ++t)
            pg[t] = __int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(p[t & 3]), g + 16 * (t >> 2)));
          float a0 = acc[g][0] * cgr, a1 = acc[g][1] * cgr;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            a0 = fmaf(pg[t], bf16_lo(Vw[u][t]), a0);
            a1 = fmaf(pg[t], bf16_hi(Vw[u][t]), a1);
          }
          acc[g][0] = a0;
          acc[g][1] = a1;
        }
      }
    }
  }

  // 4. merge the waves into this split's partial, four heads per round
  const int stride = kD + 2;
  for (int g0 = 0; g0 < G; g0 += 4) {
    if (g0) lds_barrier();   // the previous round has read red
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = g0 + gi;
      if (g < G) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int gg = 0; gg < GMAX; ++gg)
          if (gg == g) {
            a0 = acc[gg][0];
            a1 = acc[gg][1];
          }
        red[wave][gi][2 * lane] = a0;
        red[wave][gi][2 * lane + 1] = a1;
        const float mg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), g));
        const float lg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_run), g));
        if (lane == 0) {
          red[wave][gi][kD] = mg;
          red[wave][gi][kD + 1] = lg;
        }
      }
    }
    lds_barrier();
    const int gi = threadIdx.x / kD, j = threadIdx.x - gi * kD, g = g0 + gi;
    if (gi < 4 && g < G) {
      float mm = -INFINITY;
#pragma unroll
      for (int v = 0; v < kRowWaves; ++v) mm = fmaxf(mm, red[v][gi][kD]);
      float ll = 0.f, aa = 0.f;
      if (mm != -INFINITY) {
#pragma unroll
        for (int v = 0; v < kRowWaves; ++v) {
          const float cw = exp2f(red[v][gi][kD] - mm);
          ll += red[v][gi][kD + 1] * cw;
          aa += red[v][gi][j] * cw;
        }
      }
      if (out) {
        out[((int64_t)row * G + g) * kD + j] = aa * (ll > 0.f ? 1.f / ll : 0.f);
      } else {
        float* dst = part + (((int64_t)row * G + g) * n_split + s) * stride;
        dst[j] = aa;
        if (j == 0) {
          dst[kD] = mm;
          dst[kD + 1] = ll;
        }
      }
    }
  }
}

template <int GMAX>
__global__ __launch_bounds__(kRowThreads) void select_attend_kernel(
    KvArgs kv, const uint16_t* q, int G, const float* scores, const int32_t* lo_p,
    const int32_t* hi_p, int k, const uint32_t* ghist, float scale_log2, int32_t* idx,
    int32_t* count, float* part) {
  __shared__ RowSelLds L;
  __shared__ int32_t lst[kShareCap];                // this workgroup's share of the selection
  __shared__ int64_t rows_sh[kRowWaves][2][16];     // per wave: key-row offsets of two chunks
  __shared__ float red[kRowWaves][4][kD + 2];       // merge of the waves, 4 heads a round
  __shared__ int32_t tbl[kSweep / 16];              // the row's block-table entries (paged)
  __shared__ float zsh[kRowWaves][2][16];           // G = 1: the logits from the scores
  // the kSplits workgroups of a row run on one XCD and share its scores in L2
  const int vid = xcd_remap(blockIdx.x, gridDim.x);
  const int s = vid % kSplits, row = vid / kSplits;
  const int b = row / kv.H, h = row - b * kv.H;
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int n = lane & 15, g4 = lane >> 4;
  RowWindow w = row_window(lo_p, hi_p, b, kv.L_max);
  bool vec;
  const float* srow = row_base(scores, (int64_t)row * kv.L_max, w, &vec);

  // 1. the row's threshold (histogram first, then the scores)
  const uint4 gv = ((const uint4*)(ghist + (int64_t)row * kBins))[threadIdx.x];
  float fv[kGroups][4];
  row_load(srow, w, vec, 0, fv);
  // the block-table row, kept in registers until the attention needs it
  const int n_blk = kv.block_table ? kv.L_max >> 4 : 0;
  int32_t tb[kSweep / 16 / kRowThreads];
#pragma unroll
  for (int u = 0; u < kSweep / 16 / kRowThreads; ++u) {
    const int i = threadIdx.x + u * kRowThreads;
    tb[u] = i < n_blk ? kv.block_table[(int64_t)b * n_blk + i] : -1;
  }
  // the query rows (MFMA B operand of the logits), also needed only later
  bf16x8_t Qf[4];
  {
    const uint16_t* qrow = q + ((int64_t)row * G + (n < G ? n : 0)) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t v = n < G ? ld16((const char*)(qrow + 8 * (4 * j + g4))) : u32x4_t{0, 0, 0, 0};
      Qf[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  uint32_t kr[kGroups][4];
  *(uint4*)(L.hist + 4 * threadIdx.x) = gv;
  if (threadIdx.x < 256) L.dh[threadIdx.x] = 0u;
  lds_barrier();
  uint32_t T;
  int need_eq, k_sel;
  row_threshold(
      L, k, [&]() { row_keys(fv, kr); },
      [&](auto&& f) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) f(kr[g][e]);
      },
      &T, &need_eq, &k_sel);

  // 2. ranks.  Workgroup s writes idx and lists in LDS the selected keys of
  //    ranks [r0, r1), an equal share of the k_sel selected keys
  int32_t* orow = idx + (int64_t)row * k;
  int n_list;
  {
    int cg[kGroups];
    const int lt = row_counts(kr, T, cg);
    int oa, oe, ta, te;
    row_wave_offsets(L, lt, &oa, &oe, &ta, &te);
    const int r0 = (int)((int64_t)k_sel * s / kSplits);
    const int r1 = (int)((int64_t)k_sel * (s + 1) / kSplits);
    n_list = r1 - r0;
    // ranks of this wave's selected keys: [first, last)
    const int first = oa + min(oe, need_eq);
    const int last = oa + L.wa[wave] + min(oe + L.we[wave], need_eq);
    if (first < r1 && last > r0) {
      const int pos0 = w.lo - w.o + wave * kSeg + 4 * lane;
      row_emit(kr, cg, T, need_eq, oa, oe, [&](int dst, int g, int e) {
        if (dst >= r0 && dst < r1) {
          const int t = pos0 + 256 * g + e;
          orow[dst] = t;
          lst[dst - r0] = t;
        }
      });
    }
    if (s == 0) {
      const int n_sel = min(k, ta + min(te, need_eq));   // == k_sel
      for (int i = n_sel + threadIdx.x; i < k; i += kRowThreads) orow[i] = -1;
      if (threadIdx.x == 0) count[row] = n_sel;
    }
  }

  // 3. attention over the listed keys plus this workgroup's share of the
  //    always-attended tokens t < lo and t >= hi (live ones)
  const int seq = min(kv.seq_len[b], kv.L_max);
  const int a_lo = min(w.lo, seq);
  const int a_hi = max(a_lo, min(w.hi, seq));
  const int n_extra = a_lo + (seq - a_hi);
  const int x0 = (int)((int64_t)n_extra * s / kSplits);
  const int n_att = n_list + (int)((int64_t)n_extra * (s + 1) / kSplits) - x0;
#pragma unroll
  for (int u = 0; u < kSweep / 16 / kRowThreads; ++u) tbl[threadIdx.x + u * kRowThreads] = tb[u];
  lds_barrier();   // lst and tbl are complete
  attend_share<GMAX>(kv, G, row, b, h, s, kSplits, lst, n_list, x0, n_att, a_lo, a_hi, seq,
                     n_blk ? tbl : nullptr, Qf, scale_log2, part, rows_sh, red, nullptr,
                     G == 1 ? scores + (int64_t)row * kv.L_max : nullptr, zsh);
}


// ------------------------------------------ rows longer than one sweep --
// Many rows (LOCAL): one workgroup per row lists the row's candidates itself
// -- the bin of the k-th key from the scan's histogram, then one pass over
// the row's scores keeps the keys of that bin and above in LDS in position
// order (local_list_select; the row alone, fallback_select, when they would
// not fit) -- selects, and attends over the whole selection plus the sink
// and local tokens with the 16 waves of attend_share; it writes idx, count
// and the row's normalised output (no listing kernel, no split partials, no
// merge: the step is the scan and this kernel) and zeroes the row's
// histogram; every CU streams K/V rows.  Token pool (256 rows of 65,536
// slots): 67.4 us against 72.9 for the slice listing and the list-fed
// finish.  Fewer rows: after the slice listing (the exact top-k's list in the
// top-k workspace) each of a row's n_split workgroups finishes the selection
// from the list (list_select, or fallback_select when the list overflowed),
// attends over its share, and the merge zeroes the histograms and list
// counters.
constexpr int kFinishSlices = 1024;   // listing slices of a row this kernel reads
constexpr int kFinishK = kBins;       // selected keys it stages (k <= 4096)
constexpr int kLocalList = 4096;      // keys a row's own listing holds (one workgroup per row)

// SRC: where a workgroup's candidates come from -- kFromList (the slice
// listing's list), kFromRow (its own listing of the row) or kFromSegs (the
// scan's segment candidates, n_seg segments per row).
constexpr int kFromList = 0, kFromRow = 1, kFromSegs = 2;

template <int GMAX, int SRC>
__global__ __launch_bounds__(kRowThreads) void finish_attend_kernel(
    KvArgs kv, const uint16_t* q, int G, const float* scores, const int32_t* lo_p,
    const int32_t* hi_p, int k, TopkWs ws, int n_slices, float scale_log2, int32_t* idx,
    int32_t* count, float* out, int n_split, float* part, int n_seg) {
  __shared__ RowSelLds L;
  __shared__ int32_t sel[kFinishK];                 // the selection, ascending
  __shared__ uint32_t selk[kFinishK];               // and its score keys
  __shared__ int s_off[kFinishSlices + 1], s_at[kFinishSlices];
  __shared__ int klist_n;
  __shared__ int64_t rows_sh[kRowWaves][2][16];
  __shared__ union {
    float red[kRowWaves][4][kD + 2];                // the waves' merge (attention)
    struct {
      uint32_t k[kLocalList];
      int32_t p[kLocalList];
    } list;                                         // the row's own listing (selection)
  } U;
  __shared__ float zsh[kRowWaves][2][16];           // G = 1: the logits from the scores
  // n_split > 1: the row's workgroups run on one XCD (their list and scores
  // then come from its L2); the grid is padded to a multiple of 8
  const int vid = n_split > 1 ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  const int row = vid / n_split, s = vid - row * n_split;
  if (row >= kv.B * kv.H) return;
  const int b = row / kv.H, h = row - b * kv.H;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g4 = lane >> 4;
  // the query rows (MFMA B operand of the logits), needed only later
  bf16x8_t Qf[4];
  {
    const uint16_t* qrow = q + ((int64_t)row * G + (n < G ? n : 0)) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t v = n < G ? ld16((const char*)(qrow + 8 * (4 * j + g4))) : u32x4_t{0, 0, 0, 0};
      Qf[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  uint32_t* ghist = ws.hist + (int64_t)row * ws.copies * kBins;
  const uint4 gv = SRC == kFromSegs ? make_uint4(0u, 0u, 0u, 0u) : hist_bins_summed(ws, row);
  int n_sel;
  const int32_t* lst;
  const uint32_t* lk = nullptr;   // the selection's score keys (not after the fallback)
  auto keep = [&](int dst, int p, uint32_t key) {
    sel[dst] = p;
    selk[dst] = key;
  };
  n_sel = -1;
  if constexpr (SRC == kFromRow) {
    n_sel = local_list_select<kLocalList / kRowThreads>(scores, row, kv.H, kv.L_max, lo_p, hi_p, k,
                                                        gv, L, U.list.k, U.list.p, keep);
  } else if constexpr (SRC == kFromSegs) {
    n_sel = seg_select(ws, row, n_seg, k, L, keep);
  } else if (ws.meta[2 * row + 1] >= 0) {
    n_sel = list_select(ws, row, k, n_slices, gv, L, s_off, s_at, keep);
  }
  if (n_sel < 0) {
    lds_barrier();   // every thread is past its reads of L
    if constexpr (SRC == kFromSegs)
      n_sel = fallback_select_nohist(scores, row, kv.H, kv.L_max, lo_p, hi_p, k, L, klist_n);
    else
      n_sel = fallback_select(scores, row, kv.H, kv.L_max, lo_p, hi_p, k, ghist, L, klist_n, gv);
    lst = (const int32_t*)L.hist;   // the positions, ascending
  } else {
    lst = sel;
    lk = selk;
  }
  lds_barrier();
  if (s == 0) {
    int32_t* orow = idx + (int64_t)row * k;
    for (int i = threadIdx.x; i < k; i += kRowThreads) orow[i] = i < n_sel ? lst[i] : -1;
    if (threadIdx.x == 0) count[row] = n_sel;
  }
  if (SRC != kFromSegs && n_split == 1) {   // the row's only reader: zero for the next call
    if (threadIdx.x == 0) ws.ctr[(int64_t)row * kCtrStride] = 0;
    for (int cp = 0; cp < ws.copies; ++cp)
      ((uint4*)ghist)[cp * (kBins / 4) + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  }
  // this workgroup's share: selected ranks [r0, r1) and an equal share of
  // the sink and local tokens
  const RowWindow w = row_window(lo_p, hi_p, b, kv.L_max);
  const int seq = min(kv.seq_len[b], kv.L_max);
  const int a_lo = min(w.lo, seq);
  const int a_hi = max(a_lo, min(w.hi, seq));
  const int n_extra = a_lo + (seq - a_hi);
  const int r0 = (int)((int64_t)n_sel * s / n_split), r1 = (int)((int64_t)n_sel * (s + 1) / n_split);
  const int x0 = (int)((int64_t)n_extra * s / n_split);
  const int n_att = (r1 - r0) + (int)((int64_t)n_extra * (s + 1) / n_split) - x0;
  attend_share<GMAX>(kv, G, row, b, h, s, n_split, lst + r0, r1 - r0, x0, n_att, a_lo, a_hi, seq,
                     nullptr, Qf, scale_log2, part, rows_sh, U.red, n_split == 1 ? out : nullptr,
                     G == 1 ? scores + (int64_t)row * kv.L_max : nullptr, zsh,
                     lk ? lk + r0 : nullptr);
}

}  // namespace

bool select_attend_supported(const KvArgs& kv, int G) {
  return kv.bf16 && kv.v != nullptr && kv.d_k == kD && kv.d_v == kD && G >= 1 && G <= 8 &&
         row_slots_max(kv.L_max) <= kSweep;
}

size_t select_attend_partial_bytes(const KvArgs& kv, int G) {
  return (size_t)kv.B * kv.H * G * kSplits * (kD + 2) * sizeof(float);
}

hipError_t launch_select_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                const int32_t* lo, const int32_t* hi, int k, uint32_t* hist,
                                float scale, int32_t* idx, int32_t* count, float* part,
                                float* out, hipStream_t st) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(kSplits * kv.B * kv.H);   // a multiple of 8
  if (G == 1)
    select_attend_kernel<1><<<grid, kRowThreads, 0, st>>>(kv, (const uint16_t*)q, G, scores, lo, hi,
                                                          k, hist, scale_log2, idx, count, part);
  else if (G <= 4)
    select_attend_kernel<4><<<grid, kRowThreads, 0, st>>>(kv, (const uint16_t*)q, G, scores, lo, hi,
                                                          k, hist, scale_log2, idx, count, part);
  else
    select_attend_kernel<8><<<grid, kRowThreads, 0, st>>>(kv, (const uint16_t*)q, G, scores, lo, hi,
                                                          k, hist, scale_log2, idx, count, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_reduce(part, kSplits, kD, kv.H * G, kv.B, out, st, hist, G);
}

bool finish_attend_supported(const KvArgs& kv, int G, int k) {
  return finish_attend_seg_supported(kv, G, k) && row_slots_max(kv.L_max) > kSweep;
}

// The same kernel fed by the scan's segment candidates also serves rows of
// one sweep.
bool finish_attend_seg_supported(const KvArgs& kv, int G, int k) {
  return kv.bf16 && kv.v != nullptr && kv.d_k == kD && kv.d_v == kD && G >= 1 && G <= 8 &&
         k >= 1 && k <= kFinishK && topk_supported(kv.L_max) &&
         topk_listing_slices(kv.B * kv.H, kv.L_max) <= kFinishSlices;
}

// Workgroups per row: one with many rows (every CU already busy, and no
// merge kernel), else up to kFinishSplitsFew whose partials the merge adds
// (within the split partials attend_workspace_bytes reserves).
int finish_attend_splits(const KvArgs& kv, int G, int k) {
  const int rows = kv.B * kv.H;
  if (rows >= kFinishAttendMinRows) return 1;
  return std::max(1, std::min(kFinishSplitsFew, attend_num_splits(k, rows)));
}

hipError_t launch_finish_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                const int32_t* lo, const int32_t* hi, int k, void* topk_ws,
                                float scale, int32_t* idx, int32_t* count, float* out, float* part,
                                hipStream_t st, int n_seg) {
  const int rows = kv.B * kv.H;
  const TopkWs ws = TopkWs::carve(topk_ws, rows, kv.L_max);
  const int ns = topk_listing_slices(rows, kv.L_max);
  if (ns > kFinishSlices || k > kFinishK) return hipErrorInvalidValue;
  const int S = finish_attend_splits(kv, G, k);
  // the scan's segment candidates (n_seg > 0); else one workgroup per row
  // lists the row itself, several per row share the slice listing's list
  // (each of them streaming the row from L2 took the long-context GQA step
  // from 245 to 275 us: a workgroup streams 512 KB of scores at one CU's
  // rate)
  const int src = n_seg > 0 ? kFromSegs : S == 1 ? kFromRow : kFromList;
  if (src == kFromSegs && (n_seg > kSegMax || k > kSegMaxK)) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (src == kFromList) {
    e = launch_topk_listing(scores, rows, kv.H, kv.L_max, lo, hi, k, topk_ws, st);
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const uint16_t* qq = (const uint16_t*)q;
  const unsigned grid = S == 1 ? (unsigned)rows : (unsigned)((rows * S + 7) / 8 * 8);
#define SKV_FINISH(GM, SR)                                                                      \
  finish_attend_kernel<GM, SR><<<grid, kRowThreads, 0, st>>>(kv, qq, G, scores, lo, hi, k, ws, ns, \
                                                             scale_log2, idx, count, out, S, part, \
                                                             n_seg)
#define SKV_FINISH_G(GM)                                                                        \
  do {                                                                                          \
    if (src == kFromRow) SKV_FINISH(GM, kFromRow);                                             \
    else if (src == kFromSegs) SKV_FINISH(GM, kFromSegs);                                      \
    else SKV_FINISH(GM, kFromList);                                                            \
  } while (0)
  if (G == 1) SKV_FINISH_G(1);
  else if (G <= 4) SKV_FINISH_G(4);
  else SKV_FINISH_G(8);
#undef SKV_FINISH_G
#undef SKV_FINISH
  e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  if (src == kFromSegs)   // nothing of the histograms or list counters was used
    return launch_attend_reduce(part, S, kD, kv.H * G, kv.B, out, st, nullptr, G, 1, nullptr);
  return launch_attend_reduce(part, S, kD, kv.H * G, kv.B, out, st, ws.hist, G, ws.copies, ws.ctr);
}

}  // namespace skv
