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
//    16 keys, d/32 instructions cover a key row.  A wave consumes one 16-token
//    chunk (4 KB at d = 128) per step; each lane loads d/32 x 16 B.  With
//    G <= 4 the G scores of a key land in one lane (C rows 0..3), so the
//    group max needs no cross-lane traffic.
//    The scan is persistent and software pipelined (score_stream_kernel):
//    one workgroup per resident slot, each owning a contiguous range of
//    (row, chunk) work; the table entries of a row segment are staged in LDS
//    once, so no key load waits on a table load; D chunks of loads are in
//    flight per wave, and the next chunk's loads are issued between the
//    matrix instructions and the score store (which would otherwise pin
//    them, as the two pointers may alias).
//  * G = 1 and fp32 keys use the vector ALUs: 16 lanes share a key, each lane
//    owns one 16-byte piece, a wave loads 4 keys (1 KB contiguous in a pool
//    block) per instruction, and a 4-step DPP butterfly finishes each dot.
//  * Dead tokens (past seq_len, negative table entries) never read KV memory.
#include <algorithm>

#include "skv_device.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kThreads = 256;
// Tokens per workgroup of the vector-ALU scan: 256, or down to 64 while the
// grid has fewer than kTileWgs workgroups, so short rows still spread over
// the chip: a 4-wave workgroup takes 16 U tokens per load round, and a
// single 4,096-key row in 16 workgroups of 256 went through 4 dependent
// rounds per wave (11.7 us) where 64 workgroups of 64 need one.
constexpr int kTileMax = 256, kTileMin = 64, kTileWgs = 1024;
int valu_tile(const KvArgs& kv) {
  int tile = kTileMax;
  while (tile > kTileMin &&
         (int64_t)((kv.L_max + tile - 1) / tile) * kv.H * kv.B < kTileWgs)
    tile /= 2;
  return tile;
}


// Score-key histogram of the tile (top 12 bits of the order-preserving key),
// built in LDS while scoring and added into the row's global histogram: the
// first digit of the exact top-k, fused into the scan.
struct HistArgs {
  const int32_t* lo;
  const int32_t* hi;
  uint32_t* hist;   // [B*H][copies][4096]
  // survivors (threshold prefilter): keys of the window with score >= thr[row]
  // go to the row's list [row][cap] through the fill counter ctr[row * kCtrStride]
  const float* thr;
  uint32_t* lkey;
  int32_t* lpos;
  int32_t* ctr;
  int cap;
  int copies;       // histogram copies per row (topk_hist_copies)
  // segment candidates (MODE 3): row r's workgroups are r S .. r S + S - 1,
  // workgroup r S + j lists segment j of row r into the top-k workspace
  TopkWs seg;
  int seg_s, seg_m;
};

// The copy of row r's histogram that this workgroup adds into.
__device__ __forceinline__ uint32_t* hist_copy(const HistArgs& ha, int64_t r) {
  return ha.hist + (r * ha.copies + (int)(blockIdx.x % (unsigned)ha.copies)) * 4096;
}

// Survivor staging per workgroup and row segment; a segment with more is
// reported to the consumer as an overflow (its row then takes the full top-k).
constexpr int kSvCap = 2048;
constexpr int kSvOverflow = 1 << 24;

__device__ __forceinline__ void hist_add(uint32_t* lh, float s, int t, int lo, int hi) {
  uint32_t u = __float_as_uint(s);
  if (t < lo || t >= hi || (u & 0x7f800000u) == 0x7f800000u) return;
  if (u == 0x80000000u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  atomicAdd(&lh[key >> 20], 1u);
}

// The order-preserving key of a window score (0 outside the window and for
// inf / nan, which are never candidates; -0 counts as +0).
__device__ __forceinline__ uint32_t window_key(float s, int t, int lo, int hi) {
  uint32_t u = __float_as_uint(s);
  if (t < lo || t >= hi || (u & 0x7f800000u) == 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The segment's candidates (MODE 3), once lh holds the histogram of the
// segment's window keys and sk their keys (sk[i]: token tok0 + i, i < n_tok,
// 0 outside the window): the lowest bin cb such that the keys of cb and of
// every bin above fit in m slots; the keys of bins >= cb, in position order,
// go to slots [seg m, seg m + count) of row r; count and cut (cb << 20, or 0
// when every window key was listed) to the segment's entries.
__device__ __forceinline__ void seg_flush(const uint32_t* lh, const uint32_t* sk, int n_tok,
                                          int tok0, const HistArgs& ha, int64_t r, int seg,
                                          int* sh) {
  lds_barrier();   // lh and sk are complete
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = ha.seg_m;
  int c[16], ts = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 v = ((const uint4*)lh)[4 * threadIdx.x + u];
    c[4 * u] = (int)v.x;
    c[4 * u + 1] = (int)v.y;
    c[4 * u + 2] = (int)v.z;
    c[4 * u + 3] = (int)v.w;
    ts += c[4 * u] + c[4 * u + 1] + c[4 * u + 2] + c[4 * u + 3];
  }
  // this thread's 16 keys (read now, used once the cut is known)
  uint32_t kk[16];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 16 * threadIdx.x + 4 * u;
    const uint4 v = i < n_tok ? ((const uint4*)sk)[4 * threadIdx.x + u] : make_uint4(0u, 0u, 0u, 0u);
    kk[4 * u] = v.x;
    kk[4 * u + 1] = i + 1 < n_tok ? v.y : 0u;
    kk[4 * u + 2] = i + 2 < n_tok ? v.z : 0u;
    kk[4 * u + 3] = i + 3 < n_tok ? v.w : 0u;
  }
  const int incl = wave_incl_scan(ts);
  if (lane == 63) sh[wave] = incl;
  lds_barrier();
  int below = incl - ts, total = 0;   // keys in the bins below this thread's; all keys
#pragma unroll
  for (int u = 0; u < kThreads / 64; ++u) {
    if (u < wave) below += sh[u];
    total += sh[u];
  }
  if (total <= m) {
    if (threadIdx.x == 0) sh[4] = 0;
  } else {
    // the one bin where the count from the top first exceeds m
    int above = total - below - ts;
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      if (above <= m && above + c[j] > m) sh[4] = 16 * threadIdx.x + j + 1;
      above += c[j];
    }
  }
  lds_barrier();
  const uint32_t cb = (uint32_t)sh[4];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) cnt += kk[j] != 0u && (kk[j] >> 20) >= cb;
  const int ci = wave_incl_scan(cnt);
  if (lane == 63) sh[5 + wave] = ci;   // (sh[0..4] stay as read above)
  lds_barrier();
  int off = ci - cnt, listed = 0;
#pragma unroll
  for (int u = 0; u < kThreads / 64; ++u) {
    if (u < wave) off += sh[5 + u];
    listed += sh[5 + u];
  }
  const int64_t base = r * kRowList + (int64_t)seg * m;
  uint32_t* key = ha.seg.seg_key() + base;
  int32_t* pos = ha.seg.seg_pos() + base;
  if (cnt) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (kk[j] != 0u && (kk[j] >> 20) >= cb) {
        key[off] = kk[j];
        pos[off] = tok0 + 16 * threadIdx.x + j;
        ++off;
      }
  }
  if (threadIdx.x == 0) {
    ha.seg.seg_n()[r * kRowList + seg] = listed;
    ha.seg.seg_cut()[r * kRowList + seg] = cb ? cb << 20 : 0u;
  }
}

// Write a row segment's n_tok scores, staged in LDS, to dst with one burst of
// non-temporal 16-byte stores: the same scores stored as each 16-key chunk
// is finished (64 bytes per wave, spread over the whole scan between the key
// reads) cost the L = 131,072 GQA scan 10 % and the token-pool scan 8 %; as
// one burst per segment, about half of that (plain stores in the burst: the
// token-pool scan 453 against 444 us).
__device__ __forceinline__ void stage_out(const float* ss, float* dst, int n_tok) {
  lds_barrier();   // every wave's scores are staged
  if (((uintptr_t)dst & 15) == 0) {
    for (int i = 4 * threadIdx.x; i < n_tok; i += 4 * kThreads) {
      if (i + 4 <= n_tok) {
        const float4 v4 = *(const float4*)(ss + i);   // one non-temporal 16-byte store
        __builtin_nontemporal_store(v4.x, dst + i);
        __builtin_nontemporal_store(v4.y, dst + i + 1);
        __builtin_nontemporal_store(v4.z, dst + i + 2);
        __builtin_nontemporal_store(v4.w, dst + i + 3);
      } else {
        for (int e = i; e < n_tok; ++e) dst[e] = ss[e];
      }
    }
  } else {
    for (int i = threadIdx.x; i < n_tok; i += kThreads) dst[i] = ss[i];
  }
}

__device__ __forceinline__ void hist_begin(uint32_t* lh) {
  for (int i = threadIdx.x; i < 4096; i += kThreads) lh[i] = 0u;
  lds_barrier();
}

__device__ __forceinline__ void hist_flush(uint32_t* lh, uint32_t* g) {
  lds_barrier();
  for (int i = threadIdx.x; i < 4096; i += kThreads) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(&g[i], c);
  }
}

template <bool BF16, int NPL, int GMAX, int U, bool HIST>
__global__ __launch_bounds__(kThreads) void score_valu_kernel(KvArgs kv, const void* qv, int G,
                                                               float* scores, HistArgs ha,
                                                               int tile) {
  __shared__ uint32_t lh[HIST ? 4096 : 1];
  constexpr int E = BF16 ? 8 : 4;      // elements per 16-byte piece
  constexpr int ES = BF16 ? 2 : 4;     // bytes per element
  const int b = blockIdx.z, h = blockIdx.y;
  const int t_begin = blockIdx.x * tile;
  const int t_end = min(kv.L_max, t_begin + tile);
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
  if constexpr (HIST) hist_flush(lh, hist_copy(ha, (int64_t)b * kv.H + h));
}

// Persistent pipelined scan (bf16, 2 <= G <= 16, d_k = 32 * NC).  The work is
// the list of (row r = b * H + h, chunk c of 16 tokens) pairs in row-major
// order, cpr = ceil(L_max / 16) chunks per row; workgroup w owns the slice
// [N w / W, N (w + 1) / W), at most kStageEntries / (entries per chunk)
// chunks.  For each row segment of its slice the workgroup stages the
// segment's table entries in LDS, then each wave scans a contiguous quarter
// of the segment with D chunks of loads in flight.  Lanes whose token is dead
// load the query row instead (always valid memory) and their score is -inf.
constexpr int kStageEntries = 4096;
constexpr int kStageTok = kSegMaxKeys;   // staged scores per workgroup (HIST, SEG)
constexpr int kBurstTok = 1024;          // SEG: longer segments write their scores in one burst

//
// VALU (G = 1): one query row is no contraction, so the same pipeline feeds
// the vector ALUs instead: lane (n, g4) holds the query elements of its d/32
// 16-byte pieces in registers, forms a partial dot of key n, and two lane
// exchanges (lanes n, n + 16, n + 32, n + 48) complete it.
//
// MODE 1 adds the top-12-bit key histogram of the window (first digit of the
// exact top-k); MODE 2 lists the window's keys whose score reaches the row's
// predicted threshold (threshold-prefiltered top-k), staged in LDS and added
// to the row's list with one atomic per workgroup and row segment; MODE 3
// lists the segment candidates (seg_flush), their keys kept in LDS.  In
// MODES 1 and 3 a row segment is at most kStageTok tokens, and its scores
// are staged in LDS and written in one burst at its end (stage_out) — in
// MODE 3 only for segments over kBurstTok tokens.
template <int NC, int D, int GMAX, int MODE, bool VALU>
__global__ __launch_bounds__(kThreads) void score_stream_kernel(KvArgs kv, const uint16_t* q, int G,
                                                                 float* scores, HistArgs ha,
                                                                 int cpr) {
  constexpr bool HIST = MODE == 1, SURV = MODE == 2, SEG = MODE == 3;
  __shared__ __attribute__((aligned(16))) uint32_t lh[(HIST || SEG) ? 4096 : 1];
  // the row segment's scores (HIST, SEG), written out together at its end
  __shared__ __attribute__((aligned(16))) float ss[(HIST || SEG) ? kStageTok : 1];
  __shared__ __attribute__((aligned(16))) uint32_t sk[SEG ? kStageTok : 1];   // window keys (SEG)
  __shared__ int seg_sh[SEG ? 12 : 1];
  __shared__ int32_t tab[kStageEntries];
  __shared__ uint32_t svk[SURV ? kSvCap : 1];
  __shared__ int32_t svp[SURV ? kSvCap : 1];
  __shared__ int sv_n, sv_base;
  constexpr int d_k = 32 * NC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int loff = g4 * 16;   // this lane's 16-byte piece inside each 64-byte quarter
  const int64_t N = (int64_t)kv.B * kv.H * cpr;
  const int64_t w0 = N * blockIdx.x / gridDim.x, w1 = N * (blockIdx.x + 1) / gridDim.x;
  const char* kbase = (const char*)kv.k;
  const int mode = kv.token_table ? 2 : kv.block_table ? 1 : 0;   // token / block table / none
  const int per_chunk = mode == 2 ? 16 : 1;                        // staged entries per chunk
  if ((w1 - w0) * per_chunk > kStageEntries) return;               // the host never launches this
  if ((HIST || SEG) && (w1 - w0) * 16 > kStageTok) return;          // nor this

  for (int64_t wu = w0; wu < w1;) {
    const int r = (int)(wu / cpr);
    const int c_lo = (int)(wu - (int64_t)r * cpr);
    const int c_hi = (int)min((int64_t)cpr, w1 - (int64_t)r * cpr);
    wu = (int64_t)r * cpr + c_hi;
    const int b = r / kv.H, h = r - b * kv.H;
    const int n_seg = c_hi - c_lo;
    // HIST, and SEG over kBurstTok tokens: the segment's scores go out in one
    // burst at its end.  Shorter SEG segments (one long row in 256 segments
    // of 512 tokens, whose workgroups all end together) store them as they
    // go: 12.5 against 13.1 us for that row's scan.
    const bool burst = HIST || (SEG && n_seg * 16 >= kBurstTok);

    lds_barrier();   // the previous segment is done with lh and tab
    if (mode == 1) {
      const int32_t* src = kv.block_table + (int64_t)b * cpr + c_lo;
      for (int i = threadIdx.x; i < n_seg; i += kThreads) tab[i] = src[i];
    } else if (mode == 2) {
      const int32_t* src = kv.token_table + (int64_t)b * kv.L_max + (int64_t)c_lo * 16;
      for (int i = threadIdx.x; i < n_seg * 16; i += kThreads) tab[i] = src[i];
    }
    int wlo = 0, whi = 0;
    float thr = 0.f;
    if constexpr (HIST || SEG) {
      for (int i = threadIdx.x; i < 4096; i += kThreads) lh[i] = 0u;
      wlo = ha.lo[b];
      whi = ha.hi[b];
    }
    if constexpr (SURV) {
      if (threadIdx.x == 0) sv_n = 0;
      wlo = ha.lo[b];
      whi = ha.hi[b];
      thr = ha.thr[r];
    }
    lds_barrier();

    // A operand: row n = query head n of the group (zero rows for n >= G)
    const char* qrow = (const char*)(q + ((int64_t)r * G + (n < G ? n : 0)) * d_k);
    bf16x8_t A[VALU ? 1 : NC];
    float qf[VALU ? NC : 1][8];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      u32x4_t w = ld16(qrow + j * 64 + loff);
      if constexpr (VALU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[j][2 * e] = bf16_lo(w[e]);
          qf[j][2 * e + 1] = bf16_hi(w[e]);
        }
      } else {
        if (n >= G) w = u32x4_t{0, 0, 0, 0};
        A[j] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    const int live = min(kv.seq_len[b], kv.L_max);   // tokens t < live are addressable
    const int i_lo = (n_seg * wave) / 4;              // this wave's chunks, relative to c_lo
    const int n_w = (n_seg * (wave + 1)) / 4 - i_lo;
    float* srow = scores + (int64_t)r * kv.L_max;
    const int64_t hrow = (int64_t)h * 16 + n;         // row of (head h, token n) in a pool block
    u32x4_t Bm[D][NC];

    // physical key row of this lane's token in chunk i (relative to i_lo), or -1
    auto key_row = [&](int i) -> int64_t {
      const int c = i_lo + i;
      const int t = (c_lo + c) * 16 + n;
      if (t >= live) return -1;
      if (mode == 0) return (int64_t)r * kv.L_max + t;
      if (mode == 1) {
        const int e = tab[c];   // same address in every lane: one broadcast read
        return e < 0 ? -1 : (int64_t)e * kv.H * 16 + hrow;
      }
      const int slot = tab[c * 16 + n];
      return slot < 0 ? -1 : (((int64_t)(slot >> 4) * kv.H + h) * 16 + (slot & 15));
    };
    auto issue = [&](int s, int i) {
      const int64_t row = key_row(i);
      const char* p = row >= 0 ? kbase + row * (2 * d_k) : qrow;
#pragma unroll
      for (int j = 0; j < NC; ++j) Bm[s][j] = ld16(p + j * 64 + loff);
    };
    auto mfma = [&](int s) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (VALU) {
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] = fmaf(qf[j][2 * e], bf16_lo(Bm[s][j][e]), acc[e]);
            acc[e] = fmaf(qf[j][2 * e + 1], bf16_hi(Bm[s][j][e]), acc[e]);
          }
        float d = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        acc[0] = d;
      } else {
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[j], __builtin_bit_cast(bf16x8_t, Bm[s][j]),
                                                        acc, 0, 0, 0);
      }
      return acc;
    };
    // lane (n, g4) holds C[4 g4 + k][n]: query head 4 g4 + k against key n
    // (VALU: every lane of key n holds its score in element 0)
    auto finish = [&](f32x4_t acc, int i) {
      float sc;
      if constexpr (VALU) {
        sc = acc[0];
      } else if constexpr (GMAX <= 4) {
        sc = acc[0];
        if (G > 1) sc = fmaxf(sc, acc[1]);
        if (G > 2) sc = fmaxf(sc, acc[2]);
        if (G > 3) sc = fmaxf(sc, acc[3]);
      } else {
        sc = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * g4 + k < G) sc = fmaxf(sc, acc[k]);
        sc = fmaxf(sc, __shfl_xor(sc, 16, 64));
        sc = fmaxf(sc, __shfl_xor(sc, 32, 64));
      }
      const int t = (c_lo + i_lo + i) * 16 + n;
      const bool ok = key_row(i) >= 0;
      if (g4 == 0 && t < kv.L_max) {
        const float val = ok ? sc : -INFINITY;
        if constexpr (HIST) {
          ss[t - c_lo * 16] = val;
        } else if constexpr (SEG) {
          if (burst) ss[t - c_lo * 16] = val;
          else srow[t] = val;
        } else {
          srow[t] = val;
        }
        if constexpr (HIST) {
          if (ok) hist_add(lh, sc, t, wlo, whi);
        }
        if constexpr (SEG) {
          const uint32_t key = ok ? window_key(sc, t, wlo, whi) : 0u;
          if (key) atomicAdd(&lh[key >> 20], 1u);
          sk[t - c_lo * 16] = key;
        }
        if constexpr (SURV) {
          uint32_t u = __float_as_uint(sc);
          if (ok && t >= wlo && t < whi && sc >= thr && (u & 0x7f800000u) != 0x7f800000u) {
            if (u == 0x80000000u) u = 0u;
            const int i = atomicAdd(&sv_n, 1);
            if (i < kSvCap) {
              svk[i] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
              svp[i] = t;
            }
          }
        }
      }
    };

    // software pipeline: D chunks in flight; the next chunk's loads are
    // issued between the matrix instructions and the score store
    if (n_w >= D) {
#pragma unroll
      for (int s = 0; s < D; ++s) issue(s, s);
      int i0 = 0;
      for (; i0 + 2 * D <= n_w; i0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
          const f32x4_t acc = mfma(s);
          issue(s, i0 + s + D);
          finish(acc, i0 + s);
        }
      }
#pragma unroll
      for (int s = 0; s < D; ++s) {
        const f32x4_t acc = mfma(s);
        if (i0 + s + D < n_w) issue(s, i0 + s + D);
        finish(acc, i0 + s);
      }
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (i0 + D + s < n_w) finish(mfma(s), i0 + D + s);
    } else {
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (s < n_w) issue(s, s);
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (s < n_w) finish(mfma(s), s);
    }
    if (burst) stage_out(ss, srow + c_lo * 16, min(c_hi * 16, kv.L_max) - c_lo * 16);
    if constexpr (HIST) hist_flush(lh, hist_copy(ha, r));
    if constexpr (SEG)
      seg_flush(lh, sk, min(c_hi * 16, kv.L_max) - c_lo * 16, c_lo * 16, ha, r,
                (int)blockIdx.x - r * ha.seg_s, seg_sh);
    if constexpr (SURV) {
      lds_barrier();
      const int nsv = sv_n;
      if (threadIdx.x == 0)
        sv_base = nsv ? atomicAdd(&ha.ctr[(int64_t)r * kCtrStride], nsv > kSvCap ? kSvOverflow : nsv) : 0;
      lds_barrier();
      const int base = sv_base;
      for (int i = threadIdx.x; i < min(nsv, kSvCap); i += kThreads)
        if (base + i < ha.cap) {
          ha.lkey[(int64_t)r * ha.cap + base + i] = svk[i];
          ha.lpos[(int64_t)r * ha.cap + base + i] = svp[i];
        }
    }
  }
}

template <bool BF16, int NPL, int GMAX, int U>
void launch_valu_k(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                   dim3 grid, int tile, hipStream_t s) {
  if (ha.hist)
    score_valu_kernel<BF16, NPL, GMAX, U, true><<<grid, kThreads, 0, s>>>(kv, q, G, scores, ha,
                                                                          tile);
  else
    score_valu_kernel<BF16, NPL, GMAX, U, false><<<grid, kThreads, 0, s>>>(kv, q, G, scores, ha,
                                                                           tile);
}

template <bool BF16, int NPL, int GCAP>
hipError_t launch_valu(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                       dim3 grid, int tile, hipStream_t s) {
  if (G == 1)
    launch_valu_k<BF16, NPL, 1, 4>(kv, q, G, scores, ha, grid, tile, s);
  else if (GCAP >= 2 && G == 2)
    launch_valu_k<BF16, NPL, (GCAP >= 2 ? 2 : 1), 4>(kv, q, G, scores, ha, grid, tile, s);
  else if (GCAP >= 4 && G <= 4)
    launch_valu_k<BF16, NPL, (GCAP >= 4 ? 4 : 1), 2>(kv, q, G, scores, ha, grid, tile, s);
  else if (GCAP >= 8 && G <= 8)
    launch_valu_k<BF16, NPL, (GCAP >= 8 ? 8 : 1), 2>(kv, q, G, scores, ha, grid, tile, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Workgroups of `kernel` that fit on the current device at once (occupancy x
// compute units), cached per device in `cache`.
template <typename K>
int resident_wgs(K kernel, int* cache, int n_cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= n_cache) return 1024;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 1;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <int NC, int D, int GMAX, int MODE, bool VALU = false>
hipError_t launch_stream_k(const KvArgs& kv, const void* q, int G, float* scores,
                           const HistArgs& ha, hipStream_t s) {
  static int cache[64] = {0};
  auto kern = score_stream_kernel<NC, D, GMAX, MODE, VALU>;
  const int cpr = (kv.L_max + 15) / 16;
  const int64_t n_work = (int64_t)kv.B * kv.H * cpr;
  // at least 16 chunks per workgroup and at most one workgroup per resident
  // slot, unless a slice would then stage more table entries (or, with the
  // histogram, more scores) than fit in LDS
  const int64_t cap = MODE == 1 ? kStageTok / 16 : kStageEntries / (kv.token_table ? 16 : 1);
  int64_t w = std::min<int64_t>(resident_wgs(kern, cache, 64), (n_work + 15) / 16);
  // each workgroup flushes its histogram of a row with one atomic per bin it
  // holds; few long rows spread over every resident workgroup would make
  // hundreds of them contend for the same bins, so a row gets at most 256
  // workgroups per histogram copy
  if (MODE == 1) w = std::min<int64_t>(w, (int64_t)kv.B * kv.H * 256 * ha.copies);
  w = std::max<int64_t>(std::max<int64_t>(w, (n_work + cap - 1) / cap), 1);
  // segment candidates: exactly S workgroups per row, each within its row
  if (MODE == 3) w = (int64_t)kv.B * kv.H * ha.seg_s;
  if (w > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<dim3((unsigned)w), kThreads, 0, s>>>(kv, (const uint16_t*)q, G, scores, ha, cpr);
  return hipGetLastError();
}

template <int NC, int D, int MODE>
hipError_t launch_stream_m(const KvArgs& kv, const void* q, int G, float* scores,
                           const HistArgs& ha, hipStream_t s) {
  if constexpr (NC <= 8) {
    if (G == 1) return launch_stream_k<NC, D, 1, MODE, true>(kv, q, G, scores, ha, s);
  }
  if (G <= 4) return launch_stream_k<NC, D, 4, MODE>(kv, q, G, scores, ha, s);
  return launch_stream_k<NC, D, 16, MODE>(kv, q, G, scores, ha, s);
}

// Chunks in flight per wave: D, or at d = 128 two for the histogram with one
// query head and for candidate segments of at least kBurstTok tokens.  Two
// chunks leave the vector-ALU kernel (G = 1) 149 VGPRs instead of 216, so
// three waves share a SIMD instead of two: token-pool scan 443 -> 405 us; long GQA rows from
// candidates 1-2 % faster.  The plain scan is faster with four (token pool
// 463 against 523 us), and so are the MFMA histogram scan (by 1 us of 193)
// and short latency-bound segments.
template <int NC, int D>
hipError_t launch_stream(const KvArgs& kv, const void* q, int G, float* scores, const HistArgs& ha,
                         hipStream_t s) {
  constexpr int D2 = NC == 4 ? 2 : D;
  if (ha.seg_s > 0) {
    if constexpr (NC <= 8) {
      const int64_t cpr = ((int64_t)kv.L_max + 15) / 16;
      if (cpr / ha.seg_s * 16 >= kBurstTok) return launch_stream_m<NC, D2, 3>(kv, q, G, scores, ha, s);
      return launch_stream_m<NC, D, 3>(kv, q, G, scores, ha, s);
    }
    return hipErrorInvalidValue;
  }
  if (ha.lkey) {
    if constexpr (NC <= 8) return launch_stream_m<NC, D, 2>(kv, q, G, scores, ha, s);
    return hipErrorInvalidValue;
  }
  if (ha.hist) {
    if (G == 1) return launch_stream_m<NC, D2, 1>(kv, q, G, scores, ha, s);
    return launch_stream_m<NC, D, 1>(kv, q, G, scores, ha, s);
  }
  return launch_stream_m<NC, D, 0>(kv, q, G, scores, ha, s);
}

}  // namespace

hipError_t launch_score(const KvArgs& kv, const void* q, int G, float* scores, const int32_t* lo,
                        const int32_t* hi, uint32_t* hist, hipStream_t s) {
  const int tile = valu_tile(kv);
  dim3 grid((kv.L_max + tile - 1) / tile, kv.H, kv.B);
  HistArgs ha{lo, hi, hist};
  ha.copies = topk_hist_copies(kv.B * kv.H, kv.L_max);
  if (kv.bf16 && G >= 1 && G <= 16 && kv.d_k % 32 == 0 && (G >= 2 || kv.d_k <= 256)) {
    switch (kv.d_k / 32) {
      case 2: return launch_stream<2, 4>(kv, q, G, scores, ha, s);
      case 4: return launch_stream<4, 4>(kv, q, G, scores, ha, s);
      case 8: return launch_stream<8, 2>(kv, q, G, scores, ha, s);
      case 18: return launch_stream<18, 1>(kv, q, G, scores, ha, s);
      default: break;
    }
  }
  const int E = kv.bf16 ? 8 : 4;
  const int npl = (kv.d_k / E + 15) / 16;
  if (kv.bf16) {
    if (npl == 1) return launch_valu<true, 1, 8>(kv, q, G, scores, ha, grid, tile, s);
    if (npl == 2) return launch_valu<true, 2, 4>(kv, q, G, scores, ha, grid, tile, s);
    if (npl <= 5) return launch_valu<true, 5, 1>(kv, q, G, scores, ha, grid, tile, s);
  } else {
    if (npl == 1) return launch_valu<false, 1, 8>(kv, q, G, scores, ha, grid, tile, s);
    if (npl == 2) return launch_valu<false, 2, 8>(kv, q, G, scores, ha, grid, tile, s);
    if (npl <= 4) return launch_valu<false, 4, 2>(kv, q, G, scores, ha, grid, tile, s);
  }
  return hipErrorInvalidValue;
}

bool score_seg_supported(const KvArgs& kv, int G) {
  const int nc = kv.d_k / 32;
  return kv.bf16 && G >= 1 && G <= 16 && kv.d_k % 32 == 0 && (nc == 2 || nc == 4 || nc == 8) &&
         (G >= 2 || kv.d_k <= 256);
}

hipError_t launch_score_seg(const KvArgs& kv, const void* q, int G, float* scores,
                            const int32_t* lo, const int32_t* hi, void* topk_ws, int S,
                            hipStream_t s) {
  if (!score_seg_supported(kv, G) || S < 1 || S > kSegMax) return hipErrorInvalidValue;
  HistArgs ha{lo, hi, nullptr};
  ha.seg = TopkWs::carve(topk_ws, kv.B * kv.H, kv.L_max);
  ha.seg_s = S;
  ha.seg_m = kSegSlots / S;
  switch (kv.d_k / 32) {
    case 2: return launch_stream<2, 4>(kv, q, G, scores, ha, s);
    case 4: return launch_stream<4, 4>(kv, q, G, scores, ha, s);
    default: return launch_stream<8, 2>(kv, q, G, scores, ha, s);
  }
}

bool score_prefilter_supported(const KvArgs& kv, int G) {
  const int nc = kv.d_k / 32;
  return kv.bf16 && G >= 1 && G <= 16 && kv.d_k % 32 == 0 && (nc == 2 || nc == 4 || nc == 8);
}

hipError_t launch_score_prefilter(const KvArgs& kv, const void* q, int G, float* scores,
                                  const int32_t* lo, const int32_t* hi, const float* thr,
                                  uint32_t* lkey, int32_t* lpos, int32_t* ctr, int cap,
                                  hipStream_t s) {
  HistArgs ha{lo, hi, nullptr, thr, lkey, lpos, ctr, cap, 1};
  switch (kv.d_k / 32) {
    case 2: return launch_stream<2, 4>(kv, q, G, scores, ha, s);
    case 4: return launch_stream<4, 4>(kv, q, G, scores, ha, s);
    case 8: return launch_stream<8, 2>(kv, q, G, scores, ha, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
