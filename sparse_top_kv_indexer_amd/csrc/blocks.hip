// Block-summary scoring of the history (OasisKV reading notes, section 3.2,
// after Quest): per logical 16-token block and KV head, the coordinate-wise
// minimum mn and maximum mx of the block's keys; blocks are ranked by Quest's
// upper bound of q . k over the block,
//   score_j = max_g sum_i max(q_gi mn_ji, q_gi mx_ji)     (the page gives no
// formula; this is the plainest reading), the top-K blocks per KV head are
// selected exactly (ties to the lower block), and their tokens are attended
// with the sink and local tokens by sparsekv_gather_attend.
//
// gfx950 design.  Since mx >= mn coordinate-wise,
//   sum_i max(q_i mn_i, q_i mx_i) = [max(q, 0), min(q, 0)] . [mx, mn],
// one dot product over 2d dims.  So a block's summary is stored as one
// 2d-wide "key" row [mx, mn] (bf16; the extremes of bf16 keys are bf16), the
// summaries of physical block p at row ((p / 16) H + h) 16 + p % 16 of a pool
// shaped like a KV pool of 16-row blocks, and the block scan IS the token
// scan: score_stream_kernel over that pool with the block table as its
// per-token table (logical block j -> summary row of physical block
// block_table[b][j]), the query [max(q, 0), min(q, 0)] (exact in bf16), MFMA
// for GQA groups, the fused histogram; then the exact top-k over the block
// scores and an expansion of the chosen blocks into their live tokens.
// The summary scan reads 2 rows per 16-token block: 1/8 of the key bytes.
#include "skv_device.h"
#include "skv_internal.h"
#include "skv_topk.h"

namespace skv {

namespace {

// Summary row [mx, mn] of logical block j of sequence b, KV head h, by one
// wave: lane l owns dims 2l, 2l + 1; live tokens are 16 j .. min(16 j + 16,
// seq_len, L_max) - 1.  Unmapped and empty blocks are left alone.
__device__ __forceinline__ void summarize_block(const KvArgs& kv, int b, int h, int j,
                                                uint16_t* summ, int lane) {
  const int d = kv.d_k;
  const int seq = min(kv.seq_len[b], kv.L_max);
  if (16 * j >= seq || 2 * lane >= d) return;
  const int p = kv.block_table[(int64_t)b * (kv.L_max >> 4) + j];
  if (p < 0) return;
  const int nt = min(16, seq - 16 * j);
  const uint16_t* kb = (const uint16_t*)kv.k + ((int64_t)p * kv.H + h) * 16 * d + 2 * lane;
  // all 16 loads in flight at once; rows past the live ones re-read row 0,
  // which leaves the extremes unchanged
  uint32_t w[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) w[e] = *(const uint32_t*)(kb + (int64_t)(e < nt ? e : 0) * d);
  float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float a = bf16_lo(w[e]), c = bf16_hi(w[e]);
    mx0 = fmaxf(mx0, a);
    mx1 = fmaxf(mx1, c);
    mn0 = fminf(mn0, a);
    mn1 = fminf(mn1, c);
  }
  uint16_t* dst = summ + (((int64_t)(p >> 4) * kv.H + h) * 16 + (p & 15)) * (2 * d);
  *(uint32_t*)(dst + 2 * lane) = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
  *(uint32_t*)(dst + d + 2 * lane) =
      (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
}

// Grid (ceil((j1 - j0) / 4), H), 256 threads: one wave per (logical block, head).
__global__ __launch_bounds__(256) void block_summary_kernel(KvArgs kv, int b, int j0, int j1,
                                                            uint16_t* summ) {
  const int j = j0 + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j < j1) summarize_block(kv, b, blockIdx.y, j, summ, threadIdx.x & 63);
}

// Grid (B, ceil(H / 4)), 256 threads: the block holding each sequence's last
// token (the one a decode step has just appended), one wave per head.
__global__ __launch_bounds__(256) void block_summary_last_kernel(KvArgs kv, uint16_t* summ) {
  const int b = blockIdx.x, h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int seq = min(kv.seq_len[b], kv.L_max);
  if (h < kv.H && seq > 0) summarize_block(kv, b, h, (seq - 1) >> 4, summ, threadIdx.x & 63);
}

// Grid (B, ceil(H / 4)), 256 threads, before the scan of sequence b:
// wave w re-summarises, for KV head h = 4 blockIdx.y + w, the block holding
// the sequence's last token (the one a decode step has just appended);
// the workgroup writes the block queries [max(q, 0), min(q, 0)] of these
// heads' G query heads; and workgroup (b, 0) the candidate block window
// [ceil(lo / 16), floor(hi / 16)) and the number of blocks below seq_len.
__global__ __launch_bounds__(256) void block_prep_kernel(KvArgs kv, uint16_t* summ,
                                                         const uint16_t* q, int G,
                                                         const int32_t* lo, const int32_t* hi,
                                                         uint16_t* q2, int32_t* lob, int32_t* hib,
                                                         int32_t* seqb) {
  const int b = blockIdx.x, h0 = blockIdx.y * 4;
  const int d = kv.d_k;
  const int s = min(kv.seq_len[b], kv.L_max);
  const int h = h0 + (threadIdx.x >> 6);
  if (h < kv.H && s > 0) summarize_block(kv, b, h, (s - 1) >> 4, summ, threadIdx.x & 63);
  // query rows (b, h0 G) .. (b, min(h0 + 4, H) G - 1), two dims per thread
  const int n_pairs = (min(h0 + 4, kv.H) - h0) * G * (d / 2);
  const int64_t r0 = (int64_t)b * kv.H * G + (int64_t)h0 * G;
  for (int i = threadIdx.x; i < n_pairs; i += blockDim.x) {
    const int r = i / (d / 2), c = 2 * (i - r * (d / 2));
    const uint32_t v = *(const uint32_t*)(q + (r0 + r) * d + c);
    // per bf16 half: sign bit set -> negative (or -0) part, else positive part
    const uint32_t neg = ((v >> 15) & 1u) * 0xffffu | ((v >> 31) & 1u) * 0xffff0000u;
    uint16_t* row = q2 + (r0 + r) * 2 * d;
    *(uint32_t*)(row + c) = v & ~neg;
    *(uint32_t*)(row + d + c) = v & neg;
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    const int l = max(0, min(lo[b], kv.L_max)), e = max(l, min(hi[b], kv.L_max));
    const int lb = (l + 15) / 16;
    lob[b] = lb;
    hib[b] = max(lb, e / 16);
    seqb[b] = (s + 15) / 16;
  }
}

// Grid rows: tokens 16 j .. 16 j + 15 of the chosen blocks j (live ones;
// -1 elsewhere), in the blocks' ascending order.
__global__ __launch_bounds__(256) void block_expand_kernel(const int32_t* blk_idx,
                                                           const int32_t* blk_cnt, int K, int H,
                                                           const int32_t* seq_len, int L_max,
                                                           int32_t* tok) {
  const int row = blockIdx.x, b = row / H;
  const int seq = min(seq_len[b], L_max);
  const int cnt = blk_cnt[row];
  for (int i = threadIdx.x; i < 16 * K; i += blockDim.x) {
    const int u = i >> 4;
    int t = -1;
    if (u < cnt) {
      const int j = blk_idx[(int64_t)row * K + u];
      t = j * 16 + (i & 15);
      if (j < 0 || t >= seq) t = -1;
    }
    tok[(int64_t)row * 16 * K + i] = t;
  }
}

struct BlockWs {
  void* topk;
  uint16_t* q2;
  int32_t *lob, *hib, *seqb;
  static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t layout(BlockWs* w, char* base, const KvArgs& kv, int G) {
    const int rows = kv.B * kv.H;
    size_t o = 0;
    auto take = [&](size_t bytes) {
      char* p = base ? base + o : nullptr;
      o += al(bytes);
      return p;
    };
    void* tk = take(topk_workspace_bytes(rows, kv.L_max / 16));
    uint16_t* q2 = (uint16_t*)take((size_t)kv.B * kv.H * G * 2 * kv.d_k * 2);
    int32_t* lob = (int32_t*)take((size_t)kv.B * 4);
    int32_t* hib = (int32_t*)take((size_t)kv.B * 4);
    int32_t* seqb = (int32_t*)take((size_t)kv.B * 4);
    if (w) {
      w->topk = tk;
      w->q2 = q2;
      w->lob = lob;
      w->hib = hib;
      w->seqb = seqb;
    }
    return o;
  }
};

}  // namespace

bool block_summary_supported(const KvArgs& kv) {
  return kv.bf16 && kv.block == 16 && kv.block_table && !kv.token_table &&
         (kv.d_k == 32 || kv.d_k == 64 || kv.d_k == 128);
}

// The scan stages the block table 16 entries per chunk, so a row of it must
// hold whole chunks: L_max a multiple of 256.
bool block_select_supported(const KvArgs& kv, int G) {
  return block_summary_supported(kv) && G >= 1 && G <= 16 && kv.L_max % 256 == 0 &&
         topk_supported(kv.L_max / 16);
}

size_t block_select_ws_bytes(const KvArgs& kv, int G) {
  return BlockWs::layout(nullptr, nullptr, kv, G);
}

hipError_t launch_block_summaries(const KvArgs& kv, int b, int j0, int j1, void* summ,
                                  hipStream_t s) {
  if (j1 <= j0) return hipSuccess;
  block_summary_kernel<<<dim3((j1 - j0 + 3) / 4, kv.H), 256, 0, s>>>(kv, b, j0, j1,
                                                                     (uint16_t*)summ);
  return hipGetLastError();
}

hipError_t launch_block_summaries_last(const KvArgs& kv, void* summ, hipStream_t s) {
  block_summary_last_kernel<<<dim3(kv.B, (kv.H + 3) / 4), 256, 0, s>>>(kv, (uint16_t*)summ);
  return hipGetLastError();
}

hipError_t launch_block_select(const KvArgs& kv, void* summ, const void* q, int G,
                               const int32_t* lo, const int32_t* hi, int K, float* blk_scores,
                               int32_t* blk_idx, int32_t* blk_cnt, int32_t* tok_idx, void* ws,
                               hipStream_t s) {
  BlockWs w;
  BlockWs::layout(&w, (char*)ws, kv, G);
  const int rows = kv.B * kv.H, Lb = kv.L_max / 16;
  block_prep_kernel<<<dim3(kv.B, (kv.H + 3) / 4), 256, 0, s>>>(
      kv, (uint16_t*)summ, (const uint16_t*)q, G, lo, hi, w.q2, w.lob, w.hib, w.seqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the summary pool scanned like a key pool: logical block j of sequence b is
  // "token" j, its row found through the block table used as a token table
  KvArgs sk = kv;
  sk.k = summ;
  sk.v = summ;
  sk.d_k = sk.d_v = 2 * kv.d_k;
  sk.L_max = Lb;
  sk.block_table = nullptr;
  sk.token_table = kv.block_table;
  sk.seq_len = w.seqb;
  const TopkWs tw = TopkWs::carve(w.topk, rows, Lb);
  e = launch_score(sk, w.q2, G, blk_scores, w.lob, w.hib, tw.hist, s);
  if (e != hipSuccess) return e;
  e = launch_topk(blk_scores, rows, kv.H, Lb, w.lob, w.hib, K, blk_idx, blk_cnt, w.topk, true, s);
  if (e != hipSuccess) return e;
  block_expand_kernel<<<rows, 256, 0, s>>>(blk_idx, blk_cnt, K, kv.H, kv.seq_len, kv.L_max,
                                           tok_idx);
  return hipGetLastError();
}

}  // namespace skv
