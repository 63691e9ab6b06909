// S4 -- head-adaptive block selection.  WorldAttention paper, section 3.3
// "Head-level sparsity adaptation" (per head, the smallest set of key blocks
// whose cumulative attention mass passes tau_h) and appendix A.1.2 (a cheap
// coarse estimate of where the mass lies); structured summary, method step
// (5) (block pooling, coarse selection).
//
// Two kernels:
//  * pool:   mean of every B-token query block (and key block, unless the
//            gather already produced the key-block means), float32;
//  * select: one workgroup per (head, query block): pooled logits
//            qbar.kbar_j/sqrt(d), softmax over the key blocks, a bitonic sort
//            in LDS on (mass descending, block id ascending), a prefix sum of
//            the sorted masses, the first prefix that reaches tau_h, and the
//            selected ids compacted in ascending order.
// Everything is float32 and in a fixed order, so the selection is bitwise
// reproducible; no atomics.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelThreads = 256;

// grid.x = H * (nQB + nKB_to_pool): the first H*nQB workgroups pool query
// blocks, the rest pool key blocks of k_act.
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_blocks_kernel(
    const T* __restrict__ q, const T* __restrict__ k_act, int H, int B, int L, int nQB, int nKB,
    float* __restrict__ qbar, float* __restrict__ kbar) {
  constexpr int E = Vec<T>::N;
  constexpr int CPR = D / E;
  constexpr int RPP = kPoolThreads / CPR;
  __shared__ float red[kPoolThreads * E];
  const int w = blockIdx.x;
  const int t = threadIdx.x, ch = t % CPR, r0 = t / CPR;
  const T* src;
  size_t stride;  // elements between consecutive tokens
  float* dst;
  if (w < H * nQB) {
    const int h = w / nQB, i = w % nQB;
    src = q + ((size_t)i * B * H + h) * D;
    stride = (size_t)H * D;
    dst = qbar + ((size_t)h * nQB + i) * D;
  } else {
    const int u = w - H * nQB;
    const int h = u / nKB, j = u % nKB;
    src = k_act + ((size_t)h * L + (size_t)j * B) * D;
    stride = D;
    dst = kbar + ((size_t)h * nKB + j) * D;
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int row = r0; row < B; row += RPP) {
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
    const float inv = 1.f / (float)B;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[t * E + e] = s[e] * inv;
  }
}

// Block-wide inclusive scan of one float per thread (Hillis-Steele in LDS).
__device__ float block_scan_incl(float v, float* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int o = 1; o < kSelThreads; o <<= 1) {
    const float a = t >= o ? buf[t - o] : 0.f;
    __syncthreads();
    buf[t] += a;
    __syncthreads();
  }
  return buf[t];
}

__device__ int block_scan_incl_int(int v, int* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int o = 1; o < kSelThreads; o <<= 1) {
    const int a = t >= o ? buf[t - o] : 0;
    __syncthreads();
    buf[t] += a;
    __syncthreads();
  }
  return buf[t];
}

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, const float* __restrict__ tau,
    int nQB, int nKB, int n2, float scale, int32_t* __restrict__ blk_count, int32_t* __restrict__ blk_idx,
    float* __restrict__ blk_mass) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);                 // [n2] sort keys
  float* mval = reinterpret_cast<float*>(smem + (size_t)n2 * 8);     // [nKB] logits, then masses
  int* flag = reinterpret_cast<int*>(mval + nKB);                    // [nKB]
  __shared__ float q_s[D];
  __shared__ float fbuf[kSelThreads];
  __shared__ int ibuf[kSelThreads];
  __shared__ float red[kSelThreads / kWave];
  __shared__ int nsel_s;

  const int row = blockIdx.x;  // h * nQB + i
  const int h = row / nQB;
  const int t = threadIdx.x, lane = t % kWave, wv = t / kWave;
  const float th = tau[h];

  for (int c = t; c < D; c += kSelThreads) q_s[c] = qbar[(size_t)row * D + c];
  __syncthreads();

  // pooled logits
  const float* kb = kbar + (size_t)h * nKB * D;
  float lmax = -INFINITY;
  for (int j = t; j < nKB; j += kSelThreads) {
    const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)j * D);
    float s = 0.f;
#pragma unroll 8
    for (int c = 0; c < D / 4; ++c) {
      const float4 k4 = kr[c];
      s += q_s[4 * c] * k4.x + q_s[4 * c + 1] * k4.y + q_s[4 * c + 2] * k4.z + q_s[4 * c + 3] * k4.w;
    }
    s *= scale;
    mval[j] = s;
    lmax = fmaxf(lmax, s);
  }
  // block max
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
  if (lane == 0) red[wv] = lmax;
  __syncthreads();
  float gmax = red[0];
  for (int k = 1; k < kSelThreads / kWave; ++k) gmax = fmaxf(gmax, red[k]);
  __syncthreads();
  // exp and sum (per-thread sequential, then a fixed tree)
  float lsum = 0.f;
  for (int j = t; j < nKB; j += kSelThreads) {
    const float e = expf(mval[j] - gmax);
    mval[j] = e;
    lsum += e;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
  if (lane == 0) red[wv] = lsum;
  __syncthreads();
  float gsum = 0.f;
  for (int k = 0; k < kSelThreads / kWave; ++k) gsum += red[k];
  const float inv = 1.f / gsum;
  for (int j = t; j < n2; j += kSelThreads) {
    if (j < nKB) {
      const float m = mval[j] * inv;
      mval[j] = m;
      // non-negative floats order like their bit patterns; the low word puts
      // lower ids first among equal masses when sorting descending
      key[j] = ((uint64_t)__float_as_uint(m) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
      flag[j] = 0;
      if (blk_mass) blk_mass[(size_t)row * nKB + j] = m;
    } else {
      key[j] = 0;  // padding sorts last
    }
  }
  __syncthreads();

  // bitonic sort, descending
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < n2; i += kSelThreads) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint64_t a = key[i], b = key[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            key[i] = b;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  // prefix sums of the sorted masses: thread t owns a contiguous range
  const int per = (nKB + kSelThreads - 1) / kSelThreads;
  const int lo = min(nKB, t * per), hi = min(nKB, lo + per);
  float local = 0.f;
  for (int p = lo; p < hi; ++p) local += __uint_as_float((uint32_t)(key[p] >> 32));
  const float incl = block_scan_incl(local, fbuf);
  float run = incl - local;
  int first = nKB;  // first position whose prefix reaches tau
  if (th < 1.f) {
    for (int p = lo; p < hi; ++p) {
      run += __uint_as_float((uint32_t)(key[p] >> 32));
      if (run >= th) {
        first = p;
        break;
      }
    }
  }
  // minimum over threads of `first`
  int f = first;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) f = min(f, __shfl_xor(f, o));
  if (lane == 0) ibuf[wv] = f;
  __syncthreads();
  if (t == 0) {
    int m = ibuf[0];
    for (int k = 1; k < kSelThreads / kWave; ++k) m = min(m, ibuf[k]);
    nsel_s = th >= 1.f ? nKB : (m < nKB ? m + 1 : nKB);
  }
  __syncthreads();
  const int nsel = nsel_s;
  for (int p = t; p < nsel; p += kSelThreads) flag[0xFFFFFFFFu - (uint32_t)(key[p] & 0xFFFFFFFFu)] = 1;
  __syncthreads();

  // compact the selected ids in ascending order
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += flag[j];
  const int cincl = block_scan_incl_int(cnt, ibuf);
  int pos = cincl - cnt;
  int32_t* out = blk_idx + (size_t)row * nKB;
  for (int j = lo; j < hi; ++j) {
    if (flag[j]) out[pos++] = j;
  }
  __syncthreads();
  for (int p = nsel + t; p < nKB; p += kSelThreads) out[p] = -1;
  if (t == 0) blk_count[row] = nsel;
}

template <typename T, int D>
void launch_select(const Dims& s, const void* q, const void* k_act, const float* kblk_mean, const float* tau,
                   int32_t* cnt, int32_t* idx, float* mass, char* ws, const WsLayout& w, hipStream_t st) {
  float* qbar = reinterpret_cast<float*>(ws + w.sel_qbar);
  float* kbar = kblk_mean ? const_cast<float*>(kblk_mean) : reinterpret_cast<float*>(ws + w.sel_kbar);
  const int pool_k = kblk_mean ? 0 : s.nKB;
  hipLaunchKernelGGL((pool_blocks_kernel<T, D>), dim3(s.H * (s.nQB + pool_k)), dim3(kPoolThreads), 0, st,
                     reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k_act), s.H, s.B, s.L, s.nQB,
                     s.nKB, qbar, kbar);
  int n2 = 1;
  while (n2 < s.nKB) n2 <<= 1;
  const size_t smem = (size_t)n2 * 8 + (size_t)s.nKB * 8;
  hipLaunchKernelGGL((select_rows_kernel<D>), dim3(s.rows), dim3(kSelThreads), smem, st, qbar, kbar, tau,
                     s.nQB, s.nKB, n2, 1.f / sqrtf((float)s.d), cnt, idx, mass);
}

}  // namespace
}  // namespace hsa

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
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  if (s.bf16) {
    if (s.d == 128) launch_select<bf16_t, 128>(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, wsb, w, st);
    else launch_select<bf16_t, 64>(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, wsb, w, st);
  } else {
    if (s.d == 128) launch_select<float, 128>(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, wsb, w, st);
    else launch_select<float, 64>(s, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, wsb, w, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
