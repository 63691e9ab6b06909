// S4 -- head-adaptive block selection.  WorldAttention paper, section 3.3
// "Head-level sparsity adaptation" (per head, the smallest set of key blocks
// whose cumulative attention mass passes tau_h) and appendix A.1.2 (a cheap
// coarse estimate of where the mass lies); structured summary, method step
// (5) (block pooling, coarse selection).
//
// Kernels:
//  * pool:   mean of every B-token query block (and key candidate, unless the
//            gather already produced the key-block means), float32;
//  * group:  with intra-chunk keys and given key-block means, the mean of
//            each B-token history tile from its key-block means;
//  * select: pooled logits qbar.kbar_j/sqrt(d) of 16 query blocks at a time
//            on the matrix cores, then per (head, query block) one wave:
//            softmax over the key blocks, the minimal mass-ordered prefix that
//            reaches tau_h (found by a search over the mass values rather
//            than a sort), and the selected ids in ascending order.
// Everything is float32 and in a fixed order, so the selection is bitwise
// reproducible; no atomics.
#include <mutex>

#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kPoolThreads = 256;

// grid.x = H * (nQB + nC_to_pool): the first H*nQB workgroups pool query
// blocks, the rest pool the nC key candidates of k_act (candidate j < nKBh is
// the B-token history tile j, the others Bk-token blocks after the Lh history
// keys).
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_blocks_kernel(
    const T* __restrict__ q, const T* __restrict__ k_act, int H, int B, int Bk, int L, int Lh, int nQB,
    int nC, int nKBh, float* __restrict__ qbar, float* __restrict__ kbar) {
  constexpr int E = Vec<T>::N;
  constexpr int CPR = D / E;
  constexpr int RPP = kPoolThreads / CPR;
  __shared__ float red[kPoolThreads * E];
  const int w = blockIdx.x;
  const int t = threadIdx.x, ch = t % CPR, r0 = t / CPR;
  const T* src;
  size_t stride;  // elements between consecutive tokens
  float* dst;
  int n;          // tokens pooled
  if (w < H * nQB) {
    const int h = w / nQB, i = w % nQB;
    src = q + ((size_t)i * B * H + h) * D;
    stride = (size_t)H * D;
    dst = qbar + ((size_t)h * nQB + i) * D;
    n = B;
  } else {
    const int u = w - H * nQB;
    const int h = u / nC, j = u % nC;
    const size_t first = j < nKBh ? (size_t)j * B : (size_t)Lh + (size_t)(j - nKBh) * Bk;
    src = k_act + ((size_t)h * L + first) * D;
    stride = D;
    dst = kbar + ((size_t)h * nC + j) * D;
    n = j < nKBh ? B : Bk;
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int row = r0; row < n; row += RPP) {
    float f[E];
    unpack16<T>(ld16(src + row * stride + ch * E), f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[t * E + e] = acc[e];
  __syncthreads();
  if (t < CPR) {
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = 0.f;
    for (int ph = 0; ph < RPP; ++ph) {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] += red[(ph * CPR + t) * E + e];
    }
    const float inv = 1.f / (float)n;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[t * E + e] = s[e] * inv;
  }
}

// Candidate means from key-block means [H][nKB][D]: history tile j < nKBh is
// the mean of key blocks grp*j .. grp*j+grp-1 (equal sizes, so the mean of
// their means), a chunk candidate is its key block's mean.  One thread per
// (head, candidate, element).
__global__ __launch_bounds__(256) void group_means_kernel(const float* __restrict__ kblk_mean, int H, int D,
                                                          int nKB, int nC, int nKBh, int grp,
                                                          float* __restrict__ kbar) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)H * nC * D) return;
  const int e = (int)(i % D);
  const int j = (int)((i / D) % nC);
  const int h = (int)(i / ((size_t)D * nC));
  const float* src = kblk_mean + (size_t)h * nKB * D + e;
  float v;
  if (j < nKBh) {
    float acc = 0.f;
    for (int u = 0; u < grp; ++u) acc += src[(size_t)(grp * j + u) * D];
    v = acc / (float)grp;
  } else {
    v = src[(size_t)(grp * nKBh + (j - nKBh)) * D];
  }
  kbar[i] = v;
}

// Pooled logits s_ij = qbar_i . kbar_j / sqrt(d) on the float64 matrix
// cores: products of float32 values are exact in float64 and the sums round
// at 2^-53, so each logit is the float32 rounding of the exact dot product --
// the selection does not depend on a summation order.  A workgroup (4 waves)
// takes 64 key blocks x 16 query blocks of one head; wave w computes the
// 16 x 16 tile of key blocks 16*(4x + w) .. as S^T = Kbar Qbar^T (keys on
// the rows, one query per accumulator column); lane (g, c) supplies key row c
// and query column c at contraction elements 16s + 4g .. 16s + 4g + 3 of step s.
// grid (ceil(nKB/64), ceil(nQB/16), H); logits [H][nQB][nKB].
constexpr int kLogitThreads = 4 * kWave;
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kLogitThreads) void block_logits_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nQB, int nKB, float scale,
    float* __restrict__ logits) {
  const int h = blockIdx.z, q0 = blockIdx.y * 16;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4, c = lane & 15;
  const int kt = blockIdx.x * 4 + w;
  const int key = kt * 16 + c, qi = q0 + c;
  const float4* kp = reinterpret_cast<const float4*>(kbar + ((size_t)h * nKB + (key < nKB ? key : 0)) * D);
  const float4* qp = reinterpret_cast<const float4*>(qbar + ((size_t)h * nQB + (qi < nQB ? qi : 0)) * D);
  // every operand chunk is loaded before the first product (one memory latency)
  uint4 av[D / 16], bv[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    av[st] = ld16_masked(kp + 4 * st + g, key < nKB);
    bv[st] = ld16_masked(qp + 4 * st + g, qi < nQB);
  }
  f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const uint4 a = av[st], b = bv[st];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(a.x), (double)__uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(a.y), (double)__uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(a.z), (double)__uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(a.w), (double)__uint_as_float(b.w), acc, 0, 0, 0);
  }
  // the float64 16x16x4 product leaves D[g + 4i][c] in register i of lane
  // (g, c): key blocks 16*kt + g + 4i for query block q0 + c
  if (qi < nQB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = kt * 16 + g + 4 * i;
      if (kk < nKB) logits[((size_t)h * nQB + qi) * nKB + kk] = (float)(acc[i] * (double)scale);
    }
  }
}

// Selection: one wave per (head, query block) row, kSelRows rows per
// workgroup.  Lane l holds the blocks j = l + 64k in registers: softmax with
// wave-wide max and sum; then the boundary mass s_n of the minimal prefix
// (masses in decreasing order) whose sum reaches tau, found as the largest
// float bit pattern b with F(b) = sum of the masses whose bits are >= b still
// >= tau (31 halving steps; F only changes at actual masses, so b is the
// pattern of s_n).  Every block above s_n is kept, and of the blocks equal to
// s_n the lowest ids until the sum reaches tau -- the (mass descending, id
// ascending) prefix rule.  The kept ids are compacted in ascending order with
// ballots; the rest of the row is padded with -1.
constexpr int kSelRows = 4;
constexpr int kSelThreads = kSelRows * kWave;
// NPL: blocks per lane, a fixed bucket >= ceil(nKB/64) so the per-block loops
// carry no run-time guards; the padding blocks have mass 0.

// Wave-wide reductions with DPP moves (no LDS round trip): two quad
// permutations and the half-row and row mirrors leave every lane with the
// total of its 16-lane row; the four row totals are read as scalars.  The
// order is fixed, so results are reproducible.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// value of lane l of a float (the readlane builtin moves 32-bit integers)
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuadSwap1>(v);
  v += dpp_f<kQuadSwap2>(v);
  v += dpp_f<kRowHalfMirror>(v);
  v += dpp_f<kRowMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kQuadSwap1>(v));
  v = fmaxf(v, dpp_f<kQuadSwap2>(v));
  v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kRowMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ int wave_sum_int(int v) {
  v += dpp_i<kQuadSwap1>(v);
  v += dpp_i<kQuadSwap2>(v);
  v += dpp_i<kRowHalfMirror>(v);
  v += dpp_i<kRowMirror>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// The row has nKB candidates here (the caller's nC); kept candidate j < nKBh
// is written as the grp key blocks grp*j .. grp*j+grp-1, a later one as key
// block grp*nKBh + (j - nKBh) (grp = 1 and nKBh = nKB without intra-chunk
// keys); the output row holds out_stride entries.
template <int NPL>
__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(
    const float* __restrict__ logits, const float* __restrict__ tau, int rows, int nQB, int nKB, int nKBh,
    int grp, int out_stride, int32_t* __restrict__ blk_count, int32_t* __restrict__ blk_idx,
    float* __restrict__ blk_mass) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * kSelRows + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (row >= rows) return;
  const int h = row / nQB;
  const float* lr = logits + (size_t)row * nKB;

  // tau <= 0 (or NaN) keeps one block: the first prefix already reaches it
  const float th = fmaxf(tau[h], 1.17549435e-38f);
  float m[NPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int j = k * kWave + lane;
    const float v = lr[j < nKB ? j : nKB - 1];  // always issued, in bounds
    m[k] = j < nKB ? v : -INFINITY;
    lmax = fmaxf(lmax, m[k]);
  }
  const float gmax = wave_max(lmax);
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int j = k * kWave + lane;
    m[k] = j < nKB ? expf(m[k] - gmax) : 0.f;
    lsum += m[k];
  }
  const float inv = 1.f / wave_sum(lsum);
  float ltot = 0.f;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int j = k * kWave + lane;
    m[k] *= inv;  // padding blocks stay 0
    ltot += m[k];
    if (blk_mass && j < nKB) blk_mass[(size_t)row * nKB + j] = m[k];
  }
  const float total = wave_sum(ltot);

  // boundary: b_lo = largest bit pattern with F(b) >= th
  bool all = th >= 1.f || total < th;
  uint32_t b_lo = 0;
  int k_t = 0;  // tied blocks to keep
  if (!all) {
    uint32_t hi = 0x7F800000u;  // F(+inf) = 0 < th  (th > 0 here or the max is taken)
    while (hi - b_lo > 1) {
      const uint32_t mid = b_lo + ((hi - b_lo) >> 1);
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < NPL; ++k) part += __float_as_uint(m[k]) >= mid ? m[k] : 0.f;
      if (wave_sum(part) >= th) b_lo = mid;
      else hi = mid;
    }
    float sgt = 0.f;
    int nties = 0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int j = k * kWave + lane;
      const uint32_t b = __float_as_uint(m[k]);
      if (j < nKB && b > b_lo) sgt += m[k];
      if (j < nKB && b == b_lo) ++nties;
    }
    const float sum_gt = wave_sum(sgt);
    nties = wave_sum_int(nties);
    const float v = __uint_as_float(b_lo);
    int need = v > 0.f ? (int)ceilf((th - sum_gt) / v) : 1;
    k_t = max(1, min(nties, need));
  }

  // compaction in ascending id order (history tiles expand to grp key blocks)
  int32_t* out = blk_idx + (size_t)row * out_stride;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, tie_base = 0;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int j = k * kWave + lane;
    const uint32_t b = __float_as_uint(m[k]);
    const bool valid = j < nKB;
    const bool tie = valid && !all && b == b_lo;
    const uint64_t tb = __ballot(tie);
    const int tie_rank = tie_base + __popcll(tb & below);
    tie_base += __popcll(tb);
    const bool keep = valid && (all || b > b_lo || (tie && tie_rank < k_t));
    const bool hist = j < nKBh;
    const uint64_t kh = __ballot(keep && hist), kc = __ballot(keep && !hist);
    if (keep) {
      const int pos = base + grp * __popcll(kh & below) + __popcll(kc & below);
      if (hist) {
        for (int u = 0; u < grp; ++u) out[pos + u] = grp * j + u;
      } else {
        out[pos] = grp * nKBh + (j - nKBh);
      }
    }
    base += grp * __popcll(kh) + __popcll(kc);
  }
  for (int p = base + lane; p < out_stride; p += kWave) out[p] = -1;
  if (lane == 0) blk_count[row] = base;
}

template <typename T, int D>
void launch_select(const Dims& s, const void* q, const void* k_act, const float* kblk_mean, const float* tau,
                   int32_t* cnt, int32_t* idx, float* mass, char* ws, const WsLayout& w, hipStream_t st) {
  float* qbar = reinterpret_cast<float*>(ws + w.sel_qbar);
  // candidate means: the given key-block means as they are (no intra-chunk
  // keys), grouped from them, or pooled from k_act
  const bool given = kblk_mean != nullptr;
  float* kbar = given && !s.split ? const_cast<float*>(kblk_mean) : reinterpret_cast<float*>(ws + w.sel_kbar);
  const int pool_k = given ? 0 : s.nC;
  const int grp = s.B / s.Bk;
  hipLaunchKernelGGL((pool_blocks_kernel<T, D>), dim3(s.H * (s.nQB + pool_k)), dim3(kPoolThreads), 0, st,
                     reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k_act), s.H, s.B, s.Bk, s.L, s.Lh,
                     s.nQB, s.nC, s.split ? s.nKBh : s.nC, qbar, kbar);
  if (given && s.split) {
    const size_t n = (size_t)s.H * s.nC * s.d;
    hipLaunchKernelGGL(group_means_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, kblk_mean, s.H,
                       s.d, s.nKB, s.nC, s.nKBh, grp, kbar);
  }
  float* logits = reinterpret_cast<float*>(ws + w.sel_logit);
  hipLaunchKernelGGL((block_logits_kernel<D>), dim3((s.nC + 63) / 64, (s.nQB + 15) / 16, s.H), dim3(kLogitThreads),
                     0, st, qbar, kbar, s.nQB, s.nC, 1.f / sqrtf((float)s.d), logits);
  const int npl = (s.nC + kWave - 1) / kWave;
  const int nkbh = s.split ? s.nKBh : s.nC;
  const dim3 grid((s.rows + kSelRows - 1) / kSelRows);
#define HSA_SEL_CASE(N)                                                                                  \
  if (npl <= N) {                                                                                        \
    hipLaunchKernelGGL(select_rows_kernel<N>, grid, dim3(kSelThreads), 0, st, logits, tau, s.rows, s.nQB, s.nC, \
                       nkbh, grp, s.nKB, cnt, idx, mass);                                                \
    return;                                                                                              \
  }
  HSA_SEL_CASE(4)
  HSA_SEL_CASE(8)
  HSA_SEL_CASE(12)
  HSA_SEL_CASE(16)
  HSA_SEL_CASE(24)
  HSA_SEL_CASE(32)
#undef HSA_SEL_CASE
}

// Scratch of the no-allocation variant: the pooled query means, candidate
// means and pooled logits of one call, in a file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in); it passes the device address that hipGetSymbolAddress returns
// for the current device, fetched once per device.
static __device__ __align__(256) unsigned char scratch[HSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, or nullptr.
char* scratch_on_current_device(hsa_rc* rc) {
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = HSA_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *rc = HSA_ERR_HIP;
      return nullptr;
    }
    addr[dev] = static_cast<char*>(p);
  }
  return addr[dev];
}

void launch_select_any(const Dims& s, const void* q, const void* k_act, const float* kblk_mean, const float* tau,
                       int32_t* cnt, int32_t* idx, float* mass, char* ws, const WsLayout& w, hipStream_t st) {
  if (s.bf16) {
    if (s.d == 128) launch_select<bf16_t, 128>(s, q, k_act, kblk_mean, tau, cnt, idx, mass, ws, w, st);
    else launch_select<bf16_t, 64>(s, q, k_act, kblk_mean, tau, cnt, idx, mass, ws, w, st);
  } else {
    if (s.d == 128) launch_select<float, 128>(s, q, k_act, kblk_mean, tau, cnt, idx, mass, ws, w, st);
    else launch_select<float, 64>(s, q, k_act, kblk_mean, tau, cnt, idx, mass, ws, w, st);
  }
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_block_select_noalloc(const hsa_geom* geom, const void* q, const void* k_act,
                                           const float* kblk_mean, const float* tau, int32_t* blk_count,
                                           int32_t* blk_idx, float* blk_mass, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !tau || !blk_count || !blk_idx || (!k_act && !kblk_mean)) return HSA_ERR_NULL_ARG;
  const WsLayout w = ws_layout(s, 1);
  if (w.sel_end > (size_t)HSA_NOALLOC_SCRATCH_BYTES) return HSA_ERR_WORKSPACE;
  char* ws = scratch_on_current_device(&rc);
  if (!ws) return rc;
  launch_select_any(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, ws, w,
                    reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

extern "C" hsa_rc hsa_block_select(const hsa_geom* geom, const void* q, const void* k_act, const float* kblk_mean,
                                   const float* tau, int32_t* blk_count, int32_t* blk_idx, float* blk_mass,
                                   void* ws, size_t ws_bytes, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !tau || !blk_count || !blk_idx || (!k_act && !kblk_mean)) return HSA_ERR_NULL_ARG;
  const WsLayout w = ws_layout(s, 1);
  if (!ws || ws_bytes < w.sel_end) return HSA_ERR_WORKSPACE;
  launch_select_any(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, static_cast<char*>(ws), w,
                    reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
