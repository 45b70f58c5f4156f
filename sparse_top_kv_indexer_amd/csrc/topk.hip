// Exact top-k per (sequence, KV head) row of fp32 scores.
//
// What is computed: the k largest finite scores among t in [lo[b], hi[b]),
// ties broken toward the lower t, -0.0 equal to +0.0, returned as a set in
// ascending t with -1 padding (ECHO-OSDI26 wiki page, observation 5: the
// final selection is an exact top-k, whatever was prefetched).
//
// gfx950 design: a radix select on an order-preserving 32-bit key
// (sign-flipped float bits), spread over every CU.  Rows are cut into tiles
// of 4096 scores, one 256-thread workgroup per (tile, row):
//   1. hist      per-tile LDS histogram of the key's top 12 bits, added into a
//                per-row global histogram (skipped when the score scan already
//                produced it);
//   2. classify  every tile finds the bin b0 holding the k-th largest key from
//                the row histogram, counts its keys above b0 and stores its
//                keys inside b0 in its own candidate block;
//   3. write     every tile gathers its row's candidates (a few hundred keys
//                for smooth score distributions) into LDS, resolves the exact
//                32-bit threshold T with three more radix digits (8 + 8 + 4 bits),
//                decides how many keys equal to T each tile takes (lowest
//                indices first) and prefix-sums the tiles' output offsets,
//                then writes its own selected positions in index order with
//                wave ballots, so the row comes out sorted.  Resolving the
//                row redundantly in every tile costs LDS work only and saves a
//                kernel launch and a device-wide fence.
// ECHO describes an 8-bit, 256-bin histogram of the top score bits as prior
// art; a 12-bit first digit splits each fp32 octave into 8 bins, which keeps
// the threshold bin to a few hundred keys for score distributions that span a
// few octaves.  Tile 0 of the write step zeroes the row histogram, so a
// zero-filled workspace stays valid across calls.
#include "skv_device.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = kTopkTile / kThreads;      // scores per thread per tile
constexpr int kBins = 4096;
constexpr int kMaxTiles = 1024;
constexpr int kCandCap = 4096;                  // candidates resolved in LDS

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;   // inf / nan: not a candidate
  if (u == 0x80000000u) u = 0u;                        // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // finite keys are >= 0x00800000
}

struct RowWindow {
  int lo, hi, n;
};

__device__ __forceinline__ RowWindow window(const int32_t* lo_p, const int32_t* hi_p, int b,
                                            int L_max) {
  RowWindow w;
  w.lo = max(0, min(lo_p[b], L_max));
  w.hi = max(w.lo, min(hi_p[b], L_max));
  w.n = w.hi - w.lo;
  return w;
}

// Block-wide exclusive scan over 256 threads; `total` receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ex = wave_excl_scan(v, lane);
  __syncthreads();
  if (lane == 63) wsum[wave] = ex + v;
  __syncthreads();
  int before = ex;
  total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  return before;
}

// The bin holding the need-th largest entry of hist[NB] (1 <= need <= sum);
// *above_out receives the number of entries in higher bins.
template <int NB>
__device__ int find_bin(const uint32_t* hist, int need, int* above_out, int* wsum, int* pair) {
  constexpr int per = NB >= kThreads ? NB / kThreads : 1;
  const int b0 = threadIdx.x * per;
  if (threadIdx.x == 0) {
    pair[0] = 0;
    pair[1] = 0;
  }
  int tot = 0;
  if (b0 < NB) {
#pragma unroll
    for (int j = 0; j < per; ++j) tot += (int)hist[b0 + j];
  }
  int all;
  const int before = block_excl_scan(tot, wsum, all);
  int above = all - before - tot;
  if (b0 < NB) {
    for (int j = per - 1; j >= 0; --j) {
      const int c = (int)hist[b0 + j];
      if (above < need && need <= above + c) {
        pair[0] = b0 + j;
        pair[1] = above;
      }
      above += c;
    }
  }
  __syncthreads();
  const int bin = pair[0];
  *above_out = pair[1];
  __syncthreads();
  return bin;
}

// ---------------------------------------------------------------- 1. hist --
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* scores, int H, int L_max,
                                                             const int32_t* lo_p,
                                                             const int32_t* hi_p, TopkWs ws) {
  __shared__ uint32_t hist[kBins];
  const int row = blockIdx.y, tile = blockIdx.x;
  const RowWindow w = window(lo_p, hi_p, row / H, L_max);
  const int base = tile * kTopkTile;
  if (base >= w.n) return;
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  const float* s = scores + (int64_t)row * L_max + w.lo + base;
  const int cnt = min(kTopkTile, w.n - base);
  uint32_t kk[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kThreads + threadIdx.x;
    kk[u] = i < cnt ? score_key(s[i]) : 0u;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (kk[u]) atomicAdd(&hist[kk[u] >> 20], 1u);
  __syncthreads();
  uint32_t* g = ws.hist + (int64_t)row * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// ------------------------------------------------------------ 2. classify --
// Every tile finds the threshold bin b0 from the row histogram, counts its
// keys above b0 and stores its keys inside b0 in its own candidate block.
// Tile 0 also records the row's mode, b0 and counts.
__global__ __launch_bounds__(kThreads) void topk_classify_kernel(
    const float* scores, int H, int L_max, const int32_t* lo_p, const int32_t* hi_p, int k,
    int n_tiles, TopkWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ int wsum[kWaves];
  __shared__ int pair[2];
  __shared__ int s_in;
  const int row = blockIdx.y, tile = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const RowWindow w = window(lo_p, hi_p, row / H, L_max);
  const int tiles_used = max(1, (w.n + kTopkTile - 1) / kTopkTile);
  if (tile >= tiles_used) return;

  // this tile's scores and the row histogram, all loads issued together
  const int base = tile * kTopkTile;
  const int cnt = max(0, min(kTopkTile, w.n - base));
  const float* s = scores + (int64_t)row * L_max + w.lo + base;
  float sv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kThreads + threadIdx.x;
    sv[u] = i < cnt ? s[i] : -INFINITY;
  }
  stage_words<kBins / kThreads>(hist, ws.hist + (int64_t)row * kBins, kBins, threadIdx.x, kThreads);
  if (threadIdx.x == 0) s_in = 0;
  __syncthreads();
  int tot_local = 0;
#pragma unroll
  for (int j = 0; j < kBins / kThreads; ++j) tot_local += (int)hist[threadIdx.x * (kBins / kThreads) + j];
  int n_cand;
  block_excl_scan(tot_local, wsum, n_cand);
  const int k_sel = min(k, n_cand);
  // mode 0: every candidate is taken; 1: keys in bins >= b0 are taken;
  // 2: keys above b0 are taken and the threshold lies inside b0
  int mode = 0, b0 = 0, above0 = 0;
  if (k_sel < n_cand) {
    b0 = find_bin<kBins>(hist, k_sel, &above0, wsum, pair);
    mode = (k_sel - above0 == (int)hist[b0]) ? 1 : 2;
  }
  if (tile == 0 && threadIdx.x == 0) {
    int32_t* ri = ws.row_info + (int64_t)row * 4;
    ri[0] = mode;
    ri[1] = b0;
    ri[2] = above0;
    ri[3] = k_sel;
  }

  uint32_t* cand_key = ws.cand_key + ((int64_t)row * n_tiles + tile) * kTopkTile;
  int n_above = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint32_t key = score_key(sv[u]), top = key >> 20;
    const bool is_above = key != 0u && (mode == 0 || top > (uint32_t)b0 ||
                                        (mode == 1 && top == (uint32_t)b0));
    const bool is_in = mode == 2 && key != 0u && top == (uint32_t)b0;
    n_above += is_above;
    const uint64_t bm = __ballot(is_in);
    if (bm) {
      int wb = 0;
      if (lane == 0) wb = atomicAdd(&s_in, __popcll(bm));
      wb = __shfl(wb, 0, 64);
      const int slot = wb + __popcll(bm & lanemask_lt(lane));
      if (is_in) cand_key[slot] = key;
    }
  }
  int tile_above;
  block_excl_scan(n_above, wsum, tile_above);
  if (threadIdx.x == 0) {
    ws.tile_above[(int64_t)row * n_tiles + tile] = tile_above;
    ws.tile_in[(int64_t)row * n_tiles + tile] = s_in;
  }
}

// --------------------------------------------------------------- 3. write --
// Every tile resolves its row (redundantly, from the row's candidates in LDS):
// the exact threshold T, how many keys equal to T each tile takes (lowest
// indices first) and the tiles' output offsets; then it writes its own
// selected positions in index order with wave ballots.  Tile 0 also writes
// the count, pads the row with -1 and zeroes the row histogram.
__global__ __launch_bounds__(kThreads) void topk_write_kernel(const float* scores, int H, int L_max,
                                                              const int32_t* lo_p,
                                                              const int32_t* hi_p, int k,
                                                              int n_tiles, TopkWs ws,
                                                              int32_t* idx, int32_t* count) {
  __shared__ uint32_t hist[kBins];
  __shared__ int wsum[kWaves];
  __shared__ int pair[2];
  __shared__ int t_gt[kMaxTiles], t_eq[kMaxTiles], t_in[kMaxTiles], t_ab[kMaxTiles],
      t_off[kMaxTiles];
  __shared__ uint32_t c_key[kCandCap];
  __shared__ uint16_t c_tile[kCandCap];
  __shared__ int s_nc, s_off, s_take, s_nsel;
  __shared__ int wa[kWaves], we[kWaves];
  const int row = blockIdx.y, tile = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowWindow w = window(lo_p, hi_p, row / H, L_max);
  const int tiles_used = max(1, (w.n + kTopkTile - 1) / kTopkTile);
  if (tile >= tiles_used) return;
  const int base = tile * kTopkTile;
  const int cnt = max(0, min(kTopkTile, w.n - base));

  // this tile's scores (wave w owns the contiguous quarter w of the tile) and
  // the row's per-tile counts, all loads issued together
  constexpr int kSeg = kTopkTile / kWaves;
  const float* s = scores + (int64_t)row * L_max + w.lo + base;
  float sv[kSeg / 64];
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    const int i = wave * kSeg + u * 64 + lane;
    sv[u] = i < cnt ? s[i] : -INFINITY;
  }
  const int32_t* ri = ws.row_info + (int64_t)row * 4;
  const int mode = ri[0], b0 = ri[1], above0 = ri[2], k_sel = ri[3];
  for (int t = threadIdx.x; t < tiles_used; t += kThreads) {
    t_in[t] = min(ws.tile_in[(int64_t)row * n_tiles + t], kTopkTile);
    t_ab[t] = ws.tile_above[(int64_t)row * n_tiles + t];
    t_gt[t] = 0;
    t_eq[t] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0;
    for (int t = 0; t < tiles_used; ++t) {
      t_off[t] = o;
      o += t_in[t];
    }
    s_nc = o;
  }
  __syncthreads();
  const int n_c = mode == 2 ? s_nc : 0;
  const bool in_lds = n_c <= kCandCap;
  const uint32_t* ckey = ws.cand_key + (int64_t)row * n_tiles * kTopkTile;
  if (mode == 2 && in_lds) {
    for (int f0 = threadIdx.x; f0 < n_c; f0 += 8 * kThreads) {
      uint32_t kv8[8];
      int tv8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = f0 + u * kThreads;
        int t = 0;
        if (f < n_c) {            // tile of flat index f: last t with t_off[t] <= f
          int lo_t = 0, hi_t = tiles_used - 1;
          while (lo_t < hi_t) {
            const int mid = (lo_t + hi_t + 1) >> 1;
            if (t_off[mid] <= f) lo_t = mid;
            else hi_t = mid - 1;
          }
          t = lo_t;
        }
        tv8[u] = t;
        kv8[u] = f < n_c ? ckey[(int64_t)t * kTopkTile + (f - t_off[t])] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = f0 + u * kThreads;
        if (f < n_c) {
          c_key[f] = kv8[u];
          c_tile[f] = (uint16_t)tv8[u];
        }
      }
    }
  }
  __syncthreads();

  // selection: key > T, or key == T among the first t_take of each tile
  uint32_t T = 0u;
  int need_eq = 0;
  if (mode == 1) {
    T = ((uint32_t)b0 << 20) - 1u;
  } else if (mode == 2) {
    // the low 20 bits in three digits of 8, 8 and 4 bits over the few
    // candidates of the threshold bin
    int need = k_sel - above0;
    uint32_t prefix = (uint32_t)b0 << 20, mask = 0xfff00000u;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 12 : (pass == 1 ? 4 : 0);
      const uint32_t nbm = pass < 2 ? 255u : 15u;
      for (int i = threadIdx.x; i < 256; i += kThreads) hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (int f = threadIdx.x; f < n_c; f += kThreads) {
          const uint32_t key = c_key[f];
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & nbm], 1u);
        }
      } else {
        for (int t = 0; t < tiles_used; ++t)
          for (int i = threadIdx.x; i < t_in[t]; i += kThreads) {
            const uint32_t key = ckey[(int64_t)t * kTopkTile + i];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & nbm], 1u);
          }
      }
      __syncthreads();
      int above;
      const int bin = find_bin<256>(hist, need, &above, wsum, pair);
      const int in_bin = (int)hist[bin];
      need -= above;
      prefix |= (uint32_t)bin << shift;
      mask |= nbm << shift;
      if (need == in_bin) {          // the whole bin is taken
        T = prefix - 1u;
        need = 0;
        break;
      }
      T = prefix;                    // after the last digit: exact key, `need` ties
    }
    need_eq = need;
    // per-tile counts of candidates above T and equal to T
    if (in_lds) {
      for (int f = threadIdx.x; f < n_c; f += kThreads) {
        const uint32_t key = c_key[f];
        if (key > T) atomicAdd(&t_gt[c_tile[f]], 1);
        else if (key == T) atomicAdd(&t_eq[c_tile[f]], 1);
      }
    } else {
      for (int t = 0; t < tiles_used; ++t)
        for (int i = threadIdx.x; i < t_in[t]; i += kThreads) {
          const uint32_t key = ckey[(int64_t)t * kTopkTile + i];
          if (key > T) atomicAdd(&t_gt[t], 1);
          else if (key == T) atomicAdd(&t_eq[t], 1);
        }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int off = 0, eq_left = need_eq;
    for (int t = 0; t < tiles_used; ++t) {
      const int take = min(t_eq[t], eq_left);
      eq_left -= take;
      if (t == tile) {
        s_off = off;
        s_take = take;
      }
      off += t_ab[t] + t_gt[t] + take;
    }
    s_nsel = off;
  }
  __syncthreads();
  const int off = s_off, take = s_take;

  // ordered write of this tile's selected positions
  uint32_t kk[kSeg / 64];
  int ca = 0, ce = 0;
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    kk[u] = score_key(sv[u]);
    ca += __popcll(__ballot(kk[u] > T));
    ce += __popcll(__ballot(kk[u] != 0u && kk[u] == T));
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
  int32_t* orow = idx + (int64_t)row * k;
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int u = 0; u < kSeg / 64; ++u) {
    const bool is_above = kk[u] > T;
    const bool is_eq = kk[u] != 0u && kk[u] == T;
    const uint64_t ba = __ballot(is_above), be = __ballot(is_eq);
    const int a_before = oa + __popcll(ba & lt);
    const int e_before = oe + __popcll(be & lt);
    const bool sel = is_above || (is_eq && e_before < take);
    const int dst = off + a_before + min(e_before, take);
    if (sel && dst < k) orow[dst] = w.lo + base + wave * kSeg + u * 64 + lane;
    oa += __popcll(ba);
    oe += __popcll(be);
  }
  if (tile == 0) {
    const int n_sel = min(s_nsel, k);
    for (int i = n_sel + threadIdx.x; i < k; i += kThreads) orow[i] = -1;
    if (threadIdx.x == 0) count[row] = n_sel;
    uint32_t* gw = ws.hist + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kThreads) gw[i] = 0u;
  }
}

}  // namespace

size_t topk_workspace_bytes(int rows, int L_max) {
  const int n_tiles = (L_max + kTopkTile - 1) / kTopkTile;
  return TopkWs::bytes(rows, L_max, n_tiles);
}

bool topk_supported(int L_max) { return (L_max + kTopkTile - 1) / kTopkTile <= kMaxTiles; }

hipError_t launch_topk(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                       const int32_t* hi, int k, int32_t* idx, int32_t* count, void* wsp,
                       bool hist_ready, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int n_tiles = (L_max + kTopkTile - 1) / kTopkTile;
  TopkWs ws = TopkWs::carve(wsp, rows, L_max, n_tiles);
  dim3 grid(n_tiles, rows);
  if (!hist_ready) topk_hist_kernel<<<grid, kThreads, 0, s>>>(scores, H, L_max, lo, hi, ws);
  topk_classify_kernel<<<grid, kThreads, 0, s>>>(scores, H, L_max, lo, hi, k, n_tiles, ws);
  topk_write_kernel<<<grid, kThreads, 0, s>>>(scores, H, L_max, lo, hi, k, n_tiles, ws, idx,
                                              count);
  return hipGetLastError();
}

}  // namespace skv
