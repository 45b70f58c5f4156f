// Internal launch interface between the C-ABI layer (api.hip) and the kernel
// files.  Plain structs passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace skv {

struct KvArgs {
  const void* k;
  const void* v;        // nullptr => value = first d_v dims of the key row
  int bf16;             // 1: bf16 storage, 0: fp32
  int B, H, d_k, d_v;
  int block;            // 16 or 0
  int L_max;
  const int32_t* block_table;
  const int32_t* token_table;
  const int32_t* seq_len;
};

// score.hip; with hist != nullptr the scan also adds the key histogram of
// the candidates in [lo, hi) into hist [B*H][4096] (first top-k digit)
hipError_t launch_score(const KvArgs& kv, const void* q, int G, float* scores, const int32_t* lo,
                        const int32_t* hi, uint32_t* hist, hipStream_t s);

// score.hip, segment candidates: S workgroups per row, each scoring one
// segment of its row and listing the segment's highest keys into the top-k
// workspace (topk_seg_count, skv_topk.h); no histogram
bool score_seg_supported(const KvArgs& kv, int G);
hipError_t launch_score_seg(const KvArgs& kv, const void* q, int G, float* scores,
                            const int32_t* lo, const int32_t* hi, void* topk_ws, int S,
                            hipStream_t s);

// score.hip, threshold prefilter: the scan also lists, per row, the keys of
// [lo, hi) whose score is >= thr[row] (into the top-k workspace's lists)
bool score_prefilter_supported(const KvArgs& kv, int G);
hipError_t launch_score_prefilter(const KvArgs& kv, const void* q, int G, float* scores,
                                  const int32_t* lo, const int32_t* hi, const float* thr,
                                  uint32_t* lkey, int32_t* lpos, int32_t* ctr, int cap,
                                  hipStream_t s);
// topk.hip: exact top-k from those survivors (the full row when fewer than
// k survive or the list overflowed), thr updated by the EMA of the k-th score
hipError_t launch_topk_survivors(const float* scores, int rows, int H, int L_max,
                                 const int32_t* lo, const int32_t* hi, int k, int32_t* idx,
                                 int32_t* count, void* ws, float* thr, float alpha,
                                 int32_t* used_list, hipStream_t s);
bool topk_survivors_supported(int L_max);

// blocks.hip: block-summary scoring (summaries, then scan + exact top-K of
// blocks + expansion into tokens)
bool block_summary_supported(const KvArgs& kv);
bool block_select_supported(const KvArgs& kv, int G);
size_t block_select_ws_bytes(const KvArgs& kv, int G);
hipError_t launch_block_summaries(const KvArgs& kv, int b, int j0, int j1, void* summ,
                                  hipStream_t s);
hipError_t launch_block_summaries_last(const KvArgs& kv, void* summ, hipStream_t s);
hipError_t launch_block_select(const KvArgs& kv, void* summ, const void* q, int G,
                               const int32_t* lo, const int32_t* hi, int K, float* blk_scores,
                               int32_t* blk_idx, int32_t* blk_cnt, int32_t* tok_idx, void* ws,
                               hipStream_t s);

// topk.hip (workspace layout in skv_topk.h); hist_ready: the row histograms
// were already accumulated by the producer of the scores.  With map_a set,
// a selected position p of row r is written as map_b[map_a[r * map_ld + p]].
size_t topk_workspace_bytes(int rows, int L_max);
bool topk_supported(int L_max);
hipError_t launch_topk(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                       const int32_t* hi, int k, int32_t* idx, int32_t* count, void* ws,
                       bool hist_ready, hipStream_t s, const int32_t* map_a = nullptr,
                       const int32_t* map_b = nullptr, int map_ld = 0);

// topk.hip: the slice listing of rows longer than one sweep alone (after a
// scan that left the histograms in ws), for kernels that finish the
// selection themselves; topk_listing_slices = the slices per row it uses
int topk_listing_slices(int rows, int L_max);
hipError_t launch_topk_listing(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                               const int32_t* hi, int k, void* ws, hipStream_t s);

// attend.hip
int attend_num_splits(int k, int rows);
size_t attend_workspace_bytes(const KvArgs& kv, int G, int k);
hipError_t launch_gather_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                                const int32_t* lo, const int32_t* hi, float scale, float* out,
                                void* ws, size_t ws_bytes, hipStream_t s);
bool attend_supported(const KvArgs& kv, int G);
// merge of split partials [B][HG][n_split][D + 2] (acc[D], max, sum; log2
// domain) into out [B][HG][D]; with zero_hist, also zeroes each row's
// `copies` top-k histograms and (ctr != nullptr) its list counter
hipError_t launch_attend_reduce(const float* part, int n_split, int D, int HG, int B, float* out,
                                hipStream_t s, uint32_t* zero_hist = nullptr, int G = 1,
                                int copies = 1, int32_t* ctr = nullptr);

// select_attend.hip: exact top-k fused with gather + split attention (after
// launch_score with a histogram); bf16, d = 128, G <= 8, L_max <= 32768
bool select_attend_supported(const KvArgs& kv, int G);
size_t select_attend_partial_bytes(const KvArgs& kv, int G);
hipError_t launch_select_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                const int32_t* lo, const int32_t* hi, int k, uint32_t* hist,
                                float scale, int32_t* idx, int32_t* count, float* part,
                                float* out, hipStream_t s);

// select_attend.hip: rows longer than one sweep, after a scan that left the
// histograms in the top-k workspace: the slice listing, then a kernel whose
// workgroups finish the row's exact top-k (idx, count) and attend over it
// with sink and local -- one per row writing out directly when there are at
// least kFinishAttendMinRows rows (one workgroup per row streams K/V rows at
// a CU's rate, so few rows split the row over kFinishSplitsFew workgroups,
// whose partials part the merge adds) (bf16, d = 128, G <= 8, k <= 4096)
constexpr int kFinishAttendMinRows = 128;
constexpr int kFinishSplitsFew = 8;
bool finish_attend_supported(const KvArgs& kv, int G, int k);
bool finish_attend_seg_supported(const KvArgs& kv, int G, int k);
// n_seg > 0: the candidates are the segment candidates of a launch_score_seg
// with n_seg = topk_seg_count(rows, L_max, k) segments per row (no histogram)
hipError_t launch_finish_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                const int32_t* lo, const int32_t* hi, int k, void* topk_ws,
                                float scale, int32_t* idx, int32_t* count, float* out, float* part,
                                hipStream_t st, int n_seg = 0);

// mla.hip: shared-latent attention on matrix cores (v == nullptr)
bool mla_supported(const KvArgs& kv, int G);
size_t mla_workspace_bytes(const KvArgs& kv, int G, int k);
hipError_t launch_mla_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                             const int32_t* lo, const int32_t* hi, float scale, float* out,
                             void* ws, size_t ws_bytes, hipStream_t s);
// mla.hip: after a scan that left the rows' histograms in the top-k workspace
// topk_ws, the slice listing, then the exact top-k finished inside the latent
// attention kernel (idx, count written), then the merge (rows longer than one
// sweep, k <= 4096); part: mla_list_partial_bytes
bool mla_list_supported(const KvArgs& kv, int G, int k);
size_t mla_list_partial_bytes(const KvArgs& kv, int G);
// split partials the latent path of sparsekv_select_attend_resume needs
// (fused or not, whichever is larger)
size_t mla_select_attend_partial_bytes(const KvArgs& kv, int G, int k);
// (n_seg > 0: after launch_score_seg of the indexer with n_seg =
// topk_seg_count(rows, L_max, k) segments per row, no listing)
hipError_t launch_mla_list_attend(const KvArgs& kv, const void* q, int G, const float* scores,
                                  const int32_t* lo, const int32_t* hi, int k, void* topk_ws,
                                  float scale, int32_t* idx, int32_t* count, float* part,
                                  float* out, hipStream_t s, int n_seg = 0);

}  // namespace skv
