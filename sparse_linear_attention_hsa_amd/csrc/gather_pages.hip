// S2 -- active KV construction: the K_p retrieved pages, ascending id, copied
// into one contiguous head-major buffer.  WorldAttention paper, section 3.2
// "Active KV construction"; structured summary, method step (4).  With
// intra-chunk keys (section 3.3, "Inter- and intra-chunk sparse
// granularity") the current chunk's own keys and values follow the pages.
//
// One workgroup moves one B-token block of one head of one selected page (or
// of the chunk):
//  * keys   [Lp][H][d] rows -> k_act [H][L][d]   (plain copy, 16-byte chunks),
//    summing the keys of each Bk-token key block on the way (the pooled
//    block means of S4; a B-token block holds B/Bk key blocks);
//  * values [Lp][H][d] rows -> v_act [H][L/16][d][16] (16-token granules
//    stored d-major), transposed through LDS, because the PV product and the
//    low-rank projection contract over tokens and want tokens contiguous.
// All loads of a block are issued before any store so each thread keeps
// several 16-byte requests in flight (the kernel is HBM-bound).
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kBatch = 6;  // passes whose loads are in flight together

// NSUB: key blocks per B-token block (1 without intra-chunk keys, where key
// blocks are B tokens).
template <typename T, int D, int NSUB, typename Tab>
__global__ __launch_bounds__(kGatherThreads) void gather_block_kernel(
    int blk0, Tab pk, Tab pv, int n_pages, const int32_t* __restrict__ sel, const T* __restrict__ k_cur,
    const T* __restrict__ v_cur, int H, int Lp, int Kp, int B, int Bk, int L, int nKB,
    T* __restrict__ k_act, T* __restrict__ v_act, float* __restrict__ kblk_mean) {
  constexpr int E = Vec<T>::N;
  constexpr int CPR = D / E;                       // 16-byte chunks per (token, head) row
  constexpr int RPP = kGatherThreads / CPR;        // rows per pass
  constexpr int VPAD = E;                          // LDS row padding (elements)
  constexpr int VS = D + VPAD;                     // LDS row stride (elements)
  extern __shared__ __align__(16) unsigned char smem[];
  T* vs = reinterpret_cast<T*>(smem);                              // [B][VS]
  float* red = reinterpret_cast<float*>(smem + (size_t)B * VS * sizeof(T));  // [256][E]

  const int bpp = Lp / B;
  const int h = blockIdx.y;
  const int bx = blockIdx.x + blk0;  // B-token block of the active buffer
  const T* ksrc;
  const T* vsrc;
  size_t tok0, act0;  // first token of the block in its source, and in the active buffer
  if (bx < Kp * bpp) {
    const int p = bx / bpp, blk = bx % bpp;
    int page = sel ? sel[p] : p;  // no selection: the pages in table order
    page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
    ksrc = reinterpret_cast<const T*>(pk.at(page));
    vsrc = reinterpret_cast<const T*>(pv.at(page));
    tok0 = (size_t)blk * B;
    act0 = (size_t)p * Lp + tok0;
  } else {  // the chunk's own tokens, after the Kp pages
    const int blk = bx - Kp * bpp;
    ksrc = k_cur;
    vsrc = v_cur;
    tok0 = (size_t)blk * B;
    act0 = (size_t)Kp * Lp + tok0;
  }
  const int t = threadIdx.x;
  const int ch = t % CPR, r0 = t / CPR;
  const int nsub = B / Bk;
  const bool present = ksrc != nullptr && vsrc != nullptr;  // uniform: a NULL page of a device table gathers zeros

  float acc[NSUB][E];
#pragma unroll
  for (int u = 0; u < NSUB; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[u][e] = 0.f;
  const int npass = (B + RPP - 1) / RPP;
  for (int base = 0; base < npass; base += kBatch) {
    uint4 kv[kBatch], vv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int row = (base + u) * RPP + r0;
      if (base + u < npass && row < B) {
        const size_t off = ((tok0 + row) * H + h) * D + ch * E;
        if (present) {
          kv[u] = ld16_nt(ksrc + off);  // pages are read once: streaming loads
          vv[u] = ld16_nt(vsrc + off);
        } else {
          kv[u] = vv[u] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int row = (base + u) * RPP + r0;
      if (base + u < npass && row < B) {
        st16(k_act + ((size_t)h * L + act0 + row) * D + ch * E, kv[u]);
        float f[E];
        unpack16<T>(kv[u], f);
        const int sub = NSUB == 1 ? 0 : row / Bk;
#pragma unroll
        for (int su = 0; su < NSUB; ++su)
          if (su == sub)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[su][e] += f[e];
        st16(vs + row * VS + ch * E, vv[u]);
      }
    }
  }
  if (NSUB == 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) red[t * E + e] = acc[0][e];
  }
  __syncthreads();

  // values: [16 tokens][D] granules in LDS -> [D][16] granules in memory
  constexpr int PARTS = 16 / E;  // 16-byte chunks per 16-token granule row
  const int ngr = B / 16;
  const size_t g0 = act0 / 16;
  for (int c = t; c < ngr * D * PARTS; c += kGatherThreads) {
    const int gr = c / (D * PARTS);
    const int rem = c % (D * PARTS);
    const int drow = rem / PARTS, part = rem % PARTS;
    float f[E];
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = to_f32<T>(vs[(gr * 16 + part * E + e) * VS + drow]);
    st16(v_act + (((size_t)h * (L / 16) + g0 + gr) * D + drow) * 16 + part * E, pack16<T>(f));
  }

  // key-block means (fixed-order sum over the row phases), one key block at
  // a time through the same LDS area (its first one is already there when
  // a block holds one key block)
  if (kblk_mean == nullptr) return;
#pragma unroll
  for (int su = 0; su < NSUB; ++su) {
    if (su >= nsub) break;  // block-uniform
    if (NSUB > 1) {
      if (su > 0) __syncthreads();  // the previous key block's sums are read
#pragma unroll
      for (int e = 0; e < E; ++e) red[t * E + e] = acc[su][e];
      __syncthreads();
    }
    if (t < CPR) {
      float s[E];
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = 0.f;
      for (int ph = 0; ph < RPP; ++ph) {
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] += red[(ph * CPR + t) * E + e];
      }
      const float inv = 1.f / (float)Bk;
      const int j = (int)(act0 / Bk) + su;
      float* dst = kblk_mean + ((size_t)h * nKB + j) * D + t * E;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = s[e] * inv;
    }
  }
}

// chunk_only: the chunk's blocks alone (the history part stays as it is)
template <typename T, int D, typename Tab>
void launch_gather(const Dims& s, const Tab& pk, const Tab& pv, int n_pages, const int32_t* sel,
                   const void* k_cur, const void* v_cur, void* k_act, void* v_act, float* kblk_mean,
                   hipStream_t st, bool chunk_only = false) {
  constexpr int E = Vec<T>::N;
  const int nsub = s.B / s.Bk;
  const size_t smem = (size_t)s.B * (D + E) * sizeof(T) + (size_t)kGatherThreads * E * sizeof(float);
  const int hist_blocks = s.Kp * (s.Lp / s.B);
  const int blk0 = chunk_only ? hist_blocks : 0;
  dim3 grid((chunk_only ? 0 : hist_blocks) + (s.split ? s.Lq / s.B : 0), s.H);
  static_assert(HSA_MAX_INTRA_SPLIT == 4, "one instantiation per key blocks per block");
  auto kern = nsub == 1   ? gather_block_kernel<T, D, 1, Tab>
              : nsub == 2 ? gather_block_kernel<T, D, 2, Tab>
              : nsub == 3 ? gather_block_kernel<T, D, 3, Tab>
                          : gather_block_kernel<T, D, 4, Tab>;
  if (smem > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)smem);
  hipLaunchKernelGGL(kern, grid, dim3(kGatherThreads), smem, st, blk0, pk, pv, n_pages, sel,
                     reinterpret_cast<const T*>(k_cur), reinterpret_cast<const T*>(v_cur), s.H, s.Lp, s.Kp, s.B,
                     s.Bk, s.L, s.nKB, reinterpret_cast<T*>(k_act), reinterpret_cast<T*>(v_act), kblk_mean);
}

// Key-block means of the selected pages from each page's own block means
// [H][Lp/Bk][d] (written when the page was laid out): one thread per element
// of kblk_mean [H][nKB][d]; key block j is block j % bpp of page sel[j / bpp]
// (with intra-chunk keys the chunk's page-format buffers follow the history
// in sel).  A page a device table holds no means for reads as zeros.
template <typename Tab>
__global__ __launch_bounds__(256) void gather_block_means_kernel(Tab pm, int n_pages, const int32_t* __restrict__ sel,
                                                                int H, int D, int bpp, int nKB,
                                                                float* __restrict__ kblk_mean) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)H * nKB * D) return;
  const int e = (int)(i % D);
  const int j = (int)((i / D) % nKB);
  const int h = (int)(i / ((size_t)D * nKB));
  const int p = j / bpp, lb = j % bpp;
  int page = sel[p];
  page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
  const float* src = reinterpret_cast<const float*>(pm.at(page));
  kblk_mean[i] = src ? src[((size_t)h * bpp + lb) * D + e] : 0.f;
}

}  // namespace
}  // namespace hsa

namespace hsa {
namespace {

// The active-buffer gather over one page-format buffer: `tokens` tokens of
// [tokens][H][d] rows at k_src / v_src laid out as K [H][Lp][d], V
// [H][Lp/16][d][16] and Bk-token block means [H][Lp/Bk][d] (the layouts of
// the active buffer over one page; a buffer may be filled only in part).
void prepare_one(const Dims& s, int tokens, const void* k_src, const void* v_src, void* k_out, void* v_out,
                 float* blk_mean, hipStream_t st) {
  Dims one = s;
  one.split = 0;          // no chunk blocks of its own
  one.Kp = 1;
  one.Lp = tokens;        // the blocks moved
  one.L = one.Lh = s.Lp;  // the output strides: one page
  one.nKB = one.nKBh = one.nC = s.Lp / s.Bk;
  PageTable pk, pv;
  for (int j = 0; j < kMaxPages; ++j) pk.p[j] = pv.p[j] = nullptr;
  pk.p[0] = k_src;
  pv.p[0] = v_src;
  if (s.bf16) {
    if (s.d == 128) launch_gather<bf16_t, 128>(one, pk, pv, 1, nullptr, nullptr, nullptr, k_out, v_out, blk_mean, st);
    else launch_gather<bf16_t, 64>(one, pk, pv, 1, nullptr, nullptr, nullptr, k_out, v_out, blk_mean, st);
  } else {
    if (s.d == 128) launch_gather<float, 128>(one, pk, pv, 1, nullptr, nullptr, nullptr, k_out, v_out, blk_mean, st);
    else launch_gather<float, 64>(one, pk, pv, 1, nullptr, nullptr, nullptr, k_out, v_out, blk_mean, st);
  }
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_page_prepare(const hsa_geom* geom, const void* k_page, const void* v_page, void* k_out,
                                   void* v_out, float* blk_mean, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!k_page || !v_page || !k_out || !v_out) return HSA_ERR_NULL_ARG;
  prepare_one(s, s.Lp, k_page, v_page, k_out, v_out, blk_mean, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

extern "C" int32_t hsa_chunk_page_count(const hsa_geom* geom) {
  hsa::Dims s;
  if (hsa::derive(geom, &s) != HSA_OK || !s.split) return 0;
  return hsa::chunk_pages(s);
}

extern "C" hsa_rc hsa_chunk_prepare(const hsa_geom* geom, const void* k_cur, const void* v_cur,
                                    void* const* k_out, void* const* v_out, float* const* blk_mean,
                                    hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!s.split) return HSA_ERR_BAD_PARAM;
  if (!k_cur || !v_cur || !k_out || !v_out) return HSA_ERR_NULL_ARG;
  const int nc = chunk_pages(s);
  for (int j = 0; j < nc; ++j)
    if (!k_out[j] || !v_out[j]) return HSA_ERR_NULL_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t row = (size_t)s.H * s.d * s.esize;  // bytes per token of [Lq][H][d]
  for (int j = 0; j < nc; ++j) {
    const int t0 = j * s.Lp;
    const int tokens = s.Lq - t0 < s.Lp ? s.Lq - t0 : s.Lp;
    prepare_one(s, tokens, static_cast<const char*>(k_cur) + (size_t)t0 * row,
                static_cast<const char*>(v_cur) + (size_t)t0 * row, k_out[j], v_out[j],
                blk_mean ? blk_mean[j] : nullptr, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

namespace hsa {
namespace {

template <typename Tab>
hsa_rc block_means_entry(const Dims& s, const Tab& pm, int32_t n_pages, const int32_t* sel_pages, float* kblk_mean,
                         hsa_stream stream) {
  const size_t n = (size_t)s.H * s.nKB * s.d;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(gather_block_means_kernel<Tab>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pm, n_pages,
                     sel_pages, s.H, s.d, s.Lp / s.Bk, s.nKB, kblk_mean);
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_gather_block_means(const hsa_geom* geom, const float* const* page_blk_mean, int32_t n_pages,
                                         const int32_t* sel_pages, float* kblk_mean, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!page_blk_mean || !sel_pages || !kblk_mean) return HSA_ERR_NULL_ARG;
  if (n_pages < 1 || n_pages > HSA_MAX_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
  PageTable pm;
  for (int j = 0; j < kMaxPages; ++j) pm.p[j] = nullptr;
  for (int j = 0; j < n_pages; ++j) {
    if (!page_blk_mean[j]) return HSA_ERR_NULL_ARG;
    pm.p[j] = page_blk_mean[j];
  }
  return block_means_entry(s, pm, n_pages, sel_pages, kblk_mean, stream);
}

extern "C" hsa_rc hsa_gather_block_means_devtab(const hsa_geom* geom, const float* const* page_blk_mean_table,
                                                int32_t n_pages, const int32_t* sel_pages, float* kblk_mean,
                                                hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!page_blk_mean_table || !sel_pages || !kblk_mean) return HSA_ERR_NULL_ARG;
  if (n_pages < 1 || n_pages > HSA_MAX_BANK_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
  return block_means_entry(s, DevPageTable{reinterpret_cast<const void* const*>(page_blk_mean_table)}, n_pages,
                           sel_pages, kblk_mean, stream);
}

namespace hsa {
namespace {

template <typename Tab>
void gather_any(const Dims& s, const Tab& pk, const Tab& pv, int n_pages, const int32_t* sel, const void* k_cur,
                const void* v_cur, void* k_act, void* v_act, float* kblk_mean, hipStream_t st) {
  if (s.bf16) {
    if (s.d == 128) launch_gather<bf16_t, 128>(s, pk, pv, n_pages, sel, k_cur, v_cur, k_act, v_act, kblk_mean, st);
    else launch_gather<bf16_t, 64>(s, pk, pv, n_pages, sel, k_cur, v_cur, k_act, v_act, kblk_mean, st);
  } else {
    if (s.d == 128) launch_gather<float, 128>(s, pk, pv, n_pages, sel, k_cur, v_cur, k_act, v_act, kblk_mean, st);
    else launch_gather<float, 64>(s, pk, pv, n_pages, sel, k_cur, v_cur, k_act, v_act, kblk_mean, st);
  }
}

hsa_rc gather_checks(const hsa_geom* geom, Dims* s, const void* page_k, const void* page_v, int32_t n_pages,
                     int32_t max_pages, const int32_t* sel_pages, const void* k_cur, const void* v_cur, void* k_act,
                     void* v_act) {
  hsa_rc rc = derive(geom, s);
  if (rc != HSA_OK) return rc;
  if (!page_k || !page_v || !sel_pages || !k_act || !v_act) return HSA_ERR_NULL_ARG;
  if (s->split && (!k_cur || !v_cur)) return HSA_ERR_NULL_ARG;
  if (!s->split && (k_cur || v_cur)) return HSA_ERR_BAD_PARAM;
  if (n_pages < 1 || n_pages > max_pages || s->Kp > n_pages) return HSA_ERR_BAD_PARAM;
  return HSA_OK;
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_gather_active(const hsa_geom* geom, const void* const* page_k, const void* const* page_v,
                                    int32_t n_pages, const int32_t* sel_pages, const void* k_cur,
                                    const void* v_cur, void* k_act, void* v_act, float* kblk_mean,
                                    hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = gather_checks(geom, &s, page_k, page_v, n_pages, HSA_MAX_PAGES, sel_pages, k_cur, v_cur, k_act, v_act);
  if (rc != HSA_OK) return rc;
  PageTable pk, pv;
  for (int j = 0; j < kMaxPages; ++j) pk.p[j] = pv.p[j] = nullptr;
  for (int j = 0; j < n_pages; ++j) {
    if (!page_k[j] || !page_v[j]) return HSA_ERR_NULL_ARG;
    pk.p[j] = page_k[j];
    pv.p[j] = page_v[j];
  }
  gather_any(s, pk, pv, n_pages, sel_pages, k_cur, v_cur, k_act, v_act, kblk_mean,
             reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

extern "C" hsa_rc hsa_gather_active_devtab(const hsa_geom* geom, const void* const* page_k_table,
                                           const void* const* page_v_table, int32_t n_pages,
                                           const int32_t* sel_pages, const void* k_cur, const void* v_cur,
                                           void* k_act, void* v_act, float* kblk_mean, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = gather_checks(geom, &s, page_k_table, page_v_table, n_pages, HSA_MAX_BANK_PAGES, sel_pages, k_cur,
                            v_cur, k_act, v_act);
  if (rc != HSA_OK) return rc;
  gather_any(s, DevPageTable{page_k_table}, DevPageTable{page_v_table}, n_pages, sel_pages, k_cur, v_cur, k_act,
             v_act, kblk_mean, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

extern "C" hsa_rc hsa_gather_pages(const hsa_geom* geom, const void* const* page_k, const void* const* page_v,
                                   int32_t n_pages, const int32_t* sel_pages, void* k_act, void* v_act,
                                   float* kblk_mean, hsa_stream stream) {
  if (geom && geom->intra_split != 0) return HSA_ERR_BAD_PARAM;
  return hsa_gather_active(geom, page_k, page_v, n_pages, sel_pages, nullptr, nullptr, k_act, v_act, kblk_mean,
                           stream);
}

extern "C" hsa_rc hsa_gather_chunk(const hsa_geom* geom, const void* k_cur, const void* v_cur, void* k_act,
                                   void* v_act, float* kblk_mean, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!s.split) return HSA_ERR_BAD_PARAM;
  if (!k_cur || !v_cur || !k_act || !v_act) return HSA_ERR_NULL_ARG;
  PageTable none;
  for (int j = 0; j < kMaxPages; ++j) none.p[j] = nullptr;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (s.bf16) {
    if (s.d == 128) launch_gather<bf16_t, 128>(s, none, none, 1, nullptr, k_cur, v_cur, k_act, v_act, kblk_mean, st, true);
    else launch_gather<bf16_t, 64>(s, none, none, 1, nullptr, k_cur, v_cur, k_act, v_act, kblk_mean, st, true);
  } else {
    if (s.d == 128) launch_gather<float, 128>(s, none, none, 1, nullptr, k_cur, v_cur, k_act, v_act, kblk_mean, st, true);
    else launch_gather<float, 64>(s, none, none, 1, nullptr, k_cur, v_cur, k_act, v_act, kblk_mean, st, true);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
