// S1 -- page-level retrieval: mean query, mean key of every page, head-averaged
// score alpha_j = (1/H) sum_h Qbar_h . Kbar_{j,h} / sqrt(d), top-K_p pages.
// WorldAttention paper, section 3.2 "Stage 2: page-level retrieval" (score
// equation); structured summary, method step (3).
//
// HBM-bound streaming reduction.  Every page is read once, token row by token
// row (each row is H*d contiguous elements); a workgroup reduces one chunk of
// rows of one page into a float32 partial, then one workgroup per page sums
// its partials in a fixed order (bitwise reproducible), and a last small
// kernel scores and ranks the pages.
//
// Stage 1 (prompt-level retrieval, same section, "Stage 1"; section 4.5,
// ablation of candidate chunks): the cosine similarity of the current prompt
// embedding with every previous chunk's picks the top-k chunks, and the page
// scoring then runs over those chunks' pages only, K_p / k pages from each.
// The same three kernels serve it through a candidate filter: pages of other
// chunks are not read and score -inf.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kUnroll = 4;

// Column layout of one workgroup: `cols` 16-byte chunks per row handled at
// once, `par` rows in flight side by side.
struct ColMap {
  int cols, par;
};
inline ColMap col_map(int cpr) {
  ColMap m;
  m.cols = cpr < kScoreThreads ? cpr : kScoreThreads;
  m.par = kScoreThreads / m.cols;
  return m;
}

// Candidate pages: those whose chunk (page_chunk[j]) is one of the k chosen
// chunks; every page when page_chunk is null.
struct ChunkFilter {
  const int32_t* page_chunk;
  const int32_t* sel_chunks;
  int k;
};
__device__ __forceinline__ bool candidate(const ChunkFilter& f, int j) {
  if (f.page_chunk == nullptr) return true;
  const int c = f.page_chunk[j];
  bool in = false;
  for (int i = 0; i < f.k; ++i) in = in || f.sel_chunks[i] == c;
  return in;
}

template <typename T, typename Tab>
__global__ __launch_bounds__(kScoreThreads) void score_partial_kernel(
    const T* __restrict__ q, Tab pages, ChunkFilter filt, int n_pages, int Lp, int Lq, int cpr,
    int page_chunks, int page_rows, int q_rows, int mcols, int mpar, float* __restrict__ partial) {
  constexpr int E = Vec<T>::N;
  __shared__ float red[kScoreThreads * E];
  const int unit = blockIdx.x;
  const int t = threadIdx.x;
  const int col = blockIdx.y * mcols + (t % mcols);
  const int phase = t / mcols;
  const bool active = phase < mpar && col < cpr;
  const size_t row_elems = (size_t)cpr * E;

  const T* base;
  int r0, r1;
  if (unit < n_pages * page_chunks) {
    const int j = unit / page_chunks, c = unit % page_chunks;
    if (!candidate(filt, j)) return;  // a page outside the chosen chunks is not read
    base = reinterpret_cast<const T*>(pages.at(j));
    r0 = c * page_rows;
    r1 = min(Lp, r0 + page_rows);
  } else {
    const int c = unit - n_pages * page_chunks;
    base = q;
    r0 = c * q_rows;
    r1 = min(Lq, r0 + q_rows);
  }
  if (base == nullptr) return;  // non-resident page: its mean comes from the cache (whole block exits)

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (active) {
    const T* p = base + (size_t)col * E;
    int r = r0 + phase;
    for (; r + (kUnroll - 1) * mpar < r1; r += kUnroll * mpar) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = ld16_nt(p + (size_t)(r + u * mpar) * row_elems);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float f[E];
        unpack16<T>(v[u], f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += f[e];
      }
    }
    for (; r < r1; r += mpar) {
      float f[E];
      unpack16<T>(ld16_nt(p + (size_t)r * row_elems), f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[t * E + e] = acc[e];
  __syncthreads();
  if (active && phase == 0) {
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = acc[e];
    for (int ph = 1; ph < mpar; ++ph) {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] += red[(ph * mcols + (t % mcols)) * E + e];
    }
    float* out = partial + (size_t)unit * row_elems + (size_t)col * E;
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = s[e];
  }
}

// grid = (n_pages + 1, ceil(hd / 64)): 64 columns of one page per workgroup
// (the last x-index is the query buffer); thread group s (of 4) sums the
// chunk partials u = s, s+4, ... of its column, and the four sums are added
// in a fixed order (bitwise reproducible), divided by the token count.
constexpr int kMeanCols = 64;
template <typename Tab>
__global__ __launch_bounds__(kScoreThreads) void score_means_kernel(
    const float* __restrict__ partial, Tab pages, ChunkFilter filt, int n_pages, int page_chunks,
    int q_chunks, int hd, int Lp, int Lq, float* __restrict__ page_kmean, float* __restrict__ kbar,
    float* __restrict__ qbar) {
  constexpr int kGroups = kScoreThreads / kMeanCols;
  static_assert(kGroups == 4, "the final sum adds four group sums");
  __shared__ float part[kGroups][kMeanCols];
  const int j = blockIdx.x;
  const int cl = threadIdx.x % kMeanCols, grp = threadIdx.x / kMeanCols;
  const int c = blockIdx.y * kMeanCols + cl;
  const bool is_q = j == n_pages;
  if (!is_q && !candidate(filt, j)) return;  // scored -inf by the ranking kernel
  const bool resident = is_q || pages.at(j) != nullptr;  // uniform
  if (!resident) {
    // the cached mean; with no cache the page has no mean (NaN: scored -inf)
    if (grp == 0 && c < hd) kbar[(size_t)j * hd + c] = page_kmean ? page_kmean[(size_t)j * hd + c] : __builtin_nanf("");
    return;
  }
  const int n = is_q ? q_chunks : page_chunks;
  const float* p = partial + ((size_t)j * page_chunks) * hd + (c < hd ? c : 0);  // query partials follow the pages
  // eight independent sums, so eight loads are in flight per thread (the
  // query's 128 chunk partials are the longest column)
  constexpr int kAcc = 8;
  float acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.f;
  int u = grp;
  for (; u + (kAcc - 1) * kGroups < n; u += kAcc * kGroups) {
#pragma unroll
    for (int k = 0; k < kAcc; ++k) acc[k] += p[(size_t)(u + k * kGroups) * hd];
  }
#pragma unroll
  for (int k = 0; k < kAcc - 1; ++k)
    if (u + k * kGroups < n) acc[k] += p[(size_t)(u + k * kGroups) * hd];
  part[grp][cl] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (grp != 0 || c >= hd) return;
  const float m = ((part[0][cl] + part[1][cl]) + (part[2][cl] + part[3][cl])) / (float)(is_q ? Lq : Lp);
  if (is_q) {
    qbar[c] = m;
  } else {
    kbar[(size_t)j * hd + c] = m;
    if (page_kmean) page_kmean[(size_t)j * hd + c] = m;
  }
}

constexpr int kRankThreads = 1024;
constexpr int kMaxBank = HSA_MAX_BANK_PAGES;
constexpr int kRankPer = kMaxBank / kRankThreads;  // sort positions per thread
static_assert(kMaxBank % kRankThreads == 0, "whole positions per thread");
static_assert(kMaxBank <= (1 << 13), "page ids take 13 bits of the sort key");
static_assert(HSA_MAX_CHUNKS <= (1 << 12), "chunk ids take 12 bits of the sort key");

// Order-preserving code of a score, inverted so that ascending codes are
// descending scores; -0 counts as +0, so equal scores tie by id.
__device__ __forceinline__ uint64_t desc_code(float a) {
  if (a == 0.f) a = 0.f;
  const uint32_t u = __float_as_uint(a);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t)(~ord);
}

// Ascending bitonic sort of n2 (a power of two, >= 2) keys in LDS by the
// whole workgroup: every stage compares disjoint pairs (lo, lo + j).
__device__ void sort_keys(uint64_t* key, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2 / 2; i += kRankThreads) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const bool up = (lo & k) == 0;
        const uint64_t a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Exclusive prefix sum over the workgroup's 1024 threads (buf holds 16 ints).
__device__ int excl_scan_1024(int v, int* buf) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) buf[wave] = x;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < wave; ++k) before += buf[k];
  __syncthreads();
  return x - v + before;
}

// Scores and the top-K_p set of up to HSA_MAX_BANK_PAGES pages.  One wave
// per page computes the dot product in a fixed order; the pages are then
// sorted by one 64-bit key (score descending, then id ascending) and the
// first K_p are chosen; their ids are written in ascending order.
// With a chunk filter the order has three tiers: the best K_p / k pages of
// each chosen chunk, the other pages of the chosen chunks, then every other
// page (score -inf, by id); within a tier, higher score then lower id.  A
// first sort by (candidate, chunk, score, id) gives each candidate its rank
// inside its chunk, hence its tier; a second sort by (tier, score, id)
// gives the order.
__global__ __launch_bounds__(kRankThreads) void score_rank_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, ChunkFilter filt, int n_pages, int hd,
    float scale, int kp, float* __restrict__ scores, int32_t* __restrict__ sel) {
  __shared__ uint64_t key[kMaxBank];
  __shared__ unsigned char chosen[kMaxBank];
  __shared__ int buf[kRankThreads / kWave];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const bool chunked = filt.page_chunk != nullptr;
  int n2 = 2;
  while (n2 < n_pages) n2 <<= 1;
  for (int j = w; j < n_pages; j += kRankThreads / kWave) {
    const bool cand = candidate(filt, j);  // wave-uniform
    float s = 0.f;
    if (cand) {
      const float4* kb = reinterpret_cast<const float4*>(kbar + (size_t)j * hd);
      const float4* qb = reinterpret_cast<const float4*>(qbar);
      for (int c = lane; c < hd / 4; c += kWave) {
        const float4 a = qb[c], b = kb[c];
        s += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    }
    if (lane == 0) {
      // a NaN score (NaN or Inf in the inputs, or a page with neither keys
      // nor a cached mean) ranks as -inf, so the order stays total and
      // exactly K_p pages are chosen
      const float a0 = s * scale;
      const float a = cand && !__builtin_isnan(a0) ? a0 : -INFINITY;
      scores[j] = a;
      const uint64_t code = desc_code(a) << 13 | (uint64_t)j;
      // chunk ids are below HSA_MAX_CHUNKS (12 bits); the mask keeps the key well formed
      key[j] = chunked ? ((uint64_t)(cand ? 0 : 1) << 57 | (uint64_t)(filt.page_chunk[j] & 0xFFF) << 45 | code)
                       : code;
    }
  }
  for (int j = n_pages + (int)threadIdx.x; j < n2; j += kRankThreads) key[j] = ~0ull;
  __syncthreads();
  sort_keys(key, n2);
  if (chunked) {
    const int share = kp / filt.k;
    uint64_t nk[kRankPer];
#pragma unroll
    for (int m = 0; m < kRankPer; ++m) {
      const int i = (int)threadIdx.x + m * kRankThreads;
      nk[m] = ~0ull;
      if (i < n_pages) {
        const uint64_t kk = key[i];
        const uint64_t grp = kk >> 45;  // (not a candidate, chunk)
        int lo = 0, hi = i;             // first position of the group
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((key[mid] >> 45) < grp) lo = mid + 1;
          else hi = mid;
        }
        const uint64_t tier = (kk >> 57) ? 2 : (i - lo < share ? 0 : 1);
        nk[m] = tier << 45 | (kk & ((1ull << 45) - 1));
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kRankPer; ++m) {
      const int i = (int)threadIdx.x + m * kRankThreads;
      if (i < n_pages) key[i] = nk[m];
    }
    __syncthreads();
    sort_keys(key, n2);
  }
  for (int j = threadIdx.x; j < n_pages; j += kRankThreads) chosen[j] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kp; i += kRankThreads) chosen[(int)(key[i] & 0x1FFFull)] = 1;
  __syncthreads();
  // the chosen ids in ascending order: thread t owns a contiguous id range
  const int per = (n_pages + kRankThreads - 1) / kRankThreads;
  const int j0 = (int)threadIdx.x * per, j1 = min(n_pages, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += chosen[j];
  int pos = excl_scan_1024(cnt, buf);
  for (int j = j0; j < j1; ++j) {
    if (chosen[j]) {
      if (pos < kp) sel[pos] = j;
      ++pos;
    }
  }
}

// Stage 1: cosine similarity of the current prompt embedding with every
// previous chunk's (one wave per chunk, fixed-order sums), then the top-k
// chunks, ascending; a zero embedding has similarity 0.
constexpr int kRetrThreads = 1024;
__global__ __launch_bounds__(kRetrThreads) void retrieve_chunks_kernel(
    const float* __restrict__ prompt, const float* __restrict__ chunk_prompts, int n_chunks, int emb_dim,
    int k, float* __restrict__ sims, int32_t* __restrict__ sel) {
  __shared__ float sim_s[HSA_MAX_CHUNKS];
  __shared__ int chosen[HSA_MAX_CHUNKS];
  __shared__ float cur_s;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (w == 0) {
    float n = 0.f;
    for (int i = lane; i < emb_dim; i += kWave) n += prompt[i] * prompt[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
    if (lane == 0) cur_s = n;
  }
  __syncthreads();
  const float ncur = cur_s;
  for (int c = w; c < n_chunks; c += kRetrThreads / kWave) {
    const float* e = chunk_prompts + (size_t)c * emb_dim;
    float dot = 0.f, n = 0.f;
    for (int i = lane; i < emb_dim; i += kWave) {
      const float x = e[i];
      dot += prompt[i] * x;
      n += x * x;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      dot += __shfl_xor(dot, o);
      n += __shfl_xor(n, o);
    }
    if (lane == 0) {
      // a zero embedding has similarity 0 with every embedding; otherwise a
      // NaN (from NaN or Inf inputs) ranks as -inf, so the order stays total
      const float c_sim = (ncur == 0.f || n == 0.f) ? 0.f : dot / (sqrtf(ncur) * sqrtf(n));
      sim_s[c] = __builtin_isnan(c_sim) ? -INFINITY : c_sim;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n_chunks; c += kRetrThreads) {
    const float a = sim_s[c];
    int rank = 0;
    for (int i = 0; i < n_chunks; ++i) rank += sim_s[i] > a || (sim_s[i] == a && i < c);
    chosen[c] = rank < k;
    sims[c] = a;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n_chunks; c += kRetrThreads) {
    if (!chosen[c]) continue;
    int pos = 0;
    for (int i = 0; i < c; ++i) pos += chosen[i];
    if (pos < k) sel[pos] = c;
  }
}

template <typename T, typename Tab>
void launch_score(const Dims& s, const void* q, const Tab& tab, const ChunkFilter& filt, int n_pages,
                  float* page_kmean, float* scores, int32_t* sel, char* ws, const WsLayout& w, hipStream_t st) {
  const ScorePlan sp = score_plan(s, n_pages, filt.page_chunk != nullptr);
  const int cpr = s.H * s.d * s.esize / 16;
  const ColMap m = col_map(cpr);
  dim3 grid(sp.units, (cpr + m.cols - 1) / m.cols);
  float* partial = reinterpret_cast<float*>(ws + w.score_partial);
  float* qbar = reinterpret_cast<float*>(ws + w.score_qbar);
  float* kbar = reinterpret_cast<float*>(ws + w.score_kbar);
  hipLaunchKernelGGL((score_partial_kernel<T, Tab>), grid, dim3(kScoreThreads), 0, st,
                     reinterpret_cast<const T*>(q), tab, filt, n_pages, s.Lp, s.Lq, cpr, sp.page_chunks,
                     sp.page_rows, sp.q_rows, m.cols, m.par, partial);
  const int hd = s.H * s.d;
  hipLaunchKernelGGL(score_means_kernel<Tab>, dim3(n_pages + 1, (hd + kMeanCols - 1) / kMeanCols), dim3(kScoreThreads),
                     0, st, partial, tab, filt, n_pages, sp.page_chunks, sp.q_chunks, hd, s.Lp, s.Lq, page_kmean,
                     kbar, qbar);
  const float scale = 1.f / ((float)s.H * sqrtf((float)s.d));
  hipLaunchKernelGGL(score_rank_kernel, dim3(1), dim3(kRankThreads), 0, st, qbar, kbar, filt, n_pages, hd,
                     scale, s.Kp, scores, sel);
}

}  // namespace
}  // namespace hsa

namespace hsa {
namespace {

// Host table (devtab = false): n_pages <= HSA_MAX_PAGES, every entry checked
// here.  Device table (devtab = true): n_pages <= HSA_MAX_BANK_PAGES, entries
// read by the kernels.
hsa_rc score_entry(const hsa_geom* geom, const void* q, const void* const* page_k, bool devtab, float* page_kmean,
                   int32_t n_pages, const ChunkFilter& filt, float* scores, int32_t* sel_pages, void* ws,
                   size_t ws_bytes, hsa_stream stream) {
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !page_k || !scores || !sel_pages) return HSA_ERR_NULL_ARG;
  if (n_pages < 1 || n_pages > (devtab ? HSA_MAX_BANK_PAGES : HSA_MAX_PAGES) || s.Kp > n_pages)
    return HSA_ERR_BAD_PARAM;
  PageTable tab;
  if (!devtab) {
    for (int j = 0; j < kMaxPages; ++j) tab.p[j] = nullptr;
    for (int j = 0; j < n_pages; ++j) {
      tab.p[j] = page_k[j];
      if (!page_k[j] && !page_kmean) return HSA_ERR_NULL_ARG;
    }
  }
  const WsLayout w = ws_layout(s, n_pages);
  if (!ws || ws_bytes < w.total) return HSA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  const DevPageTable dtab{page_k};
  if (devtab) {
    if (s.bf16) launch_score<bf16_t>(s, q, dtab, filt, n_pages, page_kmean, scores, sel_pages, wsb, w, st);
    else launch_score<float>(s, q, dtab, filt, n_pages, page_kmean, scores, sel_pages, wsb, w, st);
  } else {
    if (s.bf16) launch_score<bf16_t>(s, q, tab, filt, n_pages, page_kmean, scores, sel_pages, wsb, w, st);
    else launch_score<float>(s, q, tab, filt, n_pages, page_kmean, scores, sel_pages, wsb, w, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

hsa_rc chunk_entry(const hsa_geom* geom, const void* q, const void* const* page_k, bool devtab, float* page_kmean,
                   int32_t n_pages, const int32_t* page_chunk, const int32_t* sel_chunks, int32_t k_chunks,
                   float* scores, int32_t* sel_pages, void* ws, size_t ws_bytes, hsa_stream stream) {
  if (!page_chunk || !sel_chunks) return HSA_ERR_NULL_ARG;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (k_chunks < 1 || k_chunks > s.Kp || s.Kp % k_chunks != 0) return HSA_ERR_BAD_PARAM;
  return score_entry(geom, q, page_k, devtab, page_kmean, n_pages, ChunkFilter{page_chunk, sel_chunks, k_chunks},
                     scores, sel_pages, ws, ws_bytes, stream);
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_score_pages(const hsa_geom* geom, const void* q, const void* const* page_k,
                                  float* page_kmean, int32_t n_pages, float* scores, int32_t* sel_pages,
                                  void* ws, size_t ws_bytes, hsa_stream stream) {
  return hsa::score_entry(geom, q, page_k, false, page_kmean, n_pages, hsa::ChunkFilter{nullptr, nullptr, 1}, scores,
                          sel_pages, ws, ws_bytes, stream);
}

extern "C" hsa_rc hsa_score_pages_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                         float* page_kmean, int32_t n_pages, float* scores, int32_t* sel_pages,
                                         void* ws, size_t ws_bytes, hsa_stream stream) {
  return hsa::score_entry(geom, q, page_k_table, true, page_kmean, n_pages, hsa::ChunkFilter{nullptr, nullptr, 1},
                          scores, sel_pages, ws, ws_bytes, stream);
}

extern "C" hsa_rc hsa_score_chunk_pages(const hsa_geom* geom, const void* q, const void* const* page_k,
                                        float* page_kmean, int32_t n_pages, const int32_t* page_chunk,
                                        const int32_t* sel_chunks, int32_t k_chunks, float* scores,
                                        int32_t* sel_pages, void* ws, size_t ws_bytes, hsa_stream stream) {
  return hsa::chunk_entry(geom, q, page_k, false, page_kmean, n_pages, page_chunk, sel_chunks, k_chunks, scores,
                          sel_pages, ws, ws_bytes, stream);
}

extern "C" hsa_rc hsa_score_chunk_pages_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                               float* page_kmean, int32_t n_pages, const int32_t* page_chunk,
                                               const int32_t* sel_chunks, int32_t k_chunks, float* scores,
                                               int32_t* sel_pages, void* ws, size_t ws_bytes, hsa_stream stream) {
  return hsa::chunk_entry(geom, q, page_k_table, true, page_kmean, n_pages, page_chunk, sel_chunks, k_chunks,
                          scores, sel_pages, ws, ws_bytes, stream);
}

extern "C" hsa_rc hsa_retrieve_chunks(const float* prompt, const float* chunk_prompts, int32_t n_chunks,
                                      int32_t emb_dim, int32_t k_chunks, float* sims, int32_t* sel_chunks,
                                      hsa_stream stream) {
  using namespace hsa;
  if (!prompt || !chunk_prompts || !sims || !sel_chunks) return HSA_ERR_NULL_ARG;
  if (n_chunks < 1 || n_chunks > HSA_MAX_CHUNKS || emb_dim < 1 || emb_dim > HSA_MAX_EMBED || k_chunks < 1 ||
      k_chunks > n_chunks)
    return HSA_ERR_BAD_PARAM;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(retrieve_chunks_kernel, dim3(1), dim3(kRetrThreads), 0, st, prompt, chunk_prompts, n_chunks,
                     emb_dim, k_chunks, sims, sel_chunks);
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
