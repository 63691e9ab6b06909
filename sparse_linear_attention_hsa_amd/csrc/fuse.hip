// S6 -- gated fusion.  WorldAttention paper, section 3.3 "Gated fusion of two
// branches"; structured summary, method step (6): gates G = X W pass through
// a sigmoid, and per head and token O = O_lin * G_lin + O_sp * G_sp.
// W has 2H output columns: column h gates the linear branch of head h and
// column H+h its sparse branch.
//
// The 16 x 2H gate logits of a 16-token tile come from the matrix cores (X rows
// and W rows are both contiguous along D), the sigmoid values go through LDS,
// then the workgroup streams O_lin / O_sp and writes O in the element type.
// HBM-bound: X, O_lin, O_sp are read once and O written once.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kFuseWaves = 8;      // per 16-token tile
constexpr int kFuseThreads = kFuseWaves * kWave;
constexpr int kMaxGateTiles = 4;   // 2H <= 64

// One workgroup (8 waves) per 16 query tokens.  The gate contraction over the
// model width is split across the waves (wave w takes every 8th step), the
// partial logits meet in LDS, and then all eight waves stream the blend.
template <typename T, int D>
__global__ __launch_bounds__(kFuseThreads) void fuse_kernel(
    const T* __restrict__ x, const T* __restrict__ w_g, const float* __restrict__ gate_override,
    const float* __restrict__ o_lin, const float* __restrict__ o_sp, int H, int Lq, T* __restrict__ out) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;
  __shared__ float part_s[kFuseWaves][16][2 * 32 + 1];
  __shared__ float gate_s[16][2 * 32];
  const int tid = threadIdx.x, wv = tid / kWave, lane = tid % kWave;
  const int g = lane >> 4, c = lane & 15;
  const int tok0 = blockIdx.x * 16;
  const int G2 = 2 * H;
  const int Dm = H * D;  // model width
  // blend geometry: 16 tokens x H heads x D, 4 floats per element; kBlendU
  // elements per thread in flight (loads from clamped, always valid
  // positions).  The first round of branch-output loads is issued before the
  // gate product, which does not need them, so the two latencies overlap.
  // Measured at 16 x 1536: 8 waves x 8 in flight 29 us, 4 x 8 33 us, 8 x 12
  // (one workgroup per CU) 35 us.
  constexpr int kBlendU = 8;
  const int per_tok = H * D / 4;
  const int total = min(16, Lq - tok0) * per_tok;
  const size_t base = (size_t)tok0 * H * D;
  float4 a[kBlendU], b[kBlendU];
  auto load_round = [&](int e0) {
#pragma unroll
    for (int u = 0; u < kBlendU; ++u) {
      const int e = min(e0 + u * kFuseThreads, total - 1);
      a[u] = reinterpret_cast<const float4*>(o_lin + base)[e];
      b[u] = reinterpret_cast<const float4*>(o_sp + base)[e];
    }
  };
  load_round(tid);
  if (x != nullptr) {
    const int ntile = (G2 + 15) / 16;
    f32x4 acc[kMaxGateTiles];
#pragma unroll
    for (int n = 0; n < kMaxGateTiles; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // G^T[col][tok] = W[col][:] . X[tok][:] ; A = W rows (gate column), B = X^T (token)
    const int tk = tok0 + c;
    const T* xr = x + (size_t)min(tk, Lq - 1) * Dm;
#pragma unroll 4
    for (int k0 = wv * KS; k0 < Dm; k0 += kFuseWaves * KS) {
      const uint4 b = ld16(xr + k0 + g * E);
#pragma unroll
      for (int n = 0; n < kMaxGateTiles; ++n) {
        if (n < ntile) {
          const int col = 16 * n + c;
          const uint4 a = ld16_masked(w_g + (size_t)min(col, G2 - 1) * Dm + k0 + g * E, col < G2);
          Mma<T>::run(acc[n], a, b);
        }
      }
    }
    // lane (g, c) holds partial G^T[16n + 4g + i][token c]
#pragma unroll
    for (int n = 0; n < kMaxGateTiles; ++n) {
      if (n < ntile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 16 * n + 4 * g + i;
          if (col < G2) part_s[wv][c][col] = acc[n][i];
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < 16 * G2; e += kFuseThreads) {
      const int tr = e / G2, col = e % G2;
      float z = 0.f;
#pragma unroll
      for (int k = 0; k < kFuseWaves; ++k) z += part_s[k][tr][col];
      gate_s[tr][col] = 1.f / (1.f + expf(-z));
    }
  } else {
    for (int e = tid; e < 16 * G2; e += kFuseThreads) {
      const int tr = e / G2, col = e % G2;
      gate_s[tr][col] = tok0 + tr < Lq ? gate_override[(size_t)(tok0 + tr) * G2 + col] : 0.f;
    }
  }
  __syncthreads();
  for (int e0 = tid; e0 < total; e0 += kBlendU * kFuseThreads) {
    if (e0 != tid) load_round(e0);
#pragma unroll
    for (int u = 0; u < kBlendU; ++u) {
      const int e = e0 + u * kFuseThreads;
      if (e < total) {
        const int tr = e / per_tok, hh = (e % per_tok) * 4 / D;
        const float gl = gate_s[tr][hh], gs = gate_s[tr][H + hh];
        const float r0 = a[u].x * gl + b[u].x * gs, r1 = a[u].y * gl + b[u].y * gs;
        const float r2 = a[u].z * gl + b[u].z * gs, r3 = a[u].w * gl + b[u].w * gs;
        if constexpr (sizeof(T) == 4) {
          reinterpret_cast<float4*>(out + base)[e] = make_float4(r0, r1, r2, r3);
        } else {
          reinterpret_cast<uint2*>(out + base)[e] = make_uint2(pack2_bf16(r0, r1), pack2_bf16(r2, r3));
        }
      }
    }
  }
}

template <typename T, int D>
void launch_fuse(const Dims& s, const void* x, const void* w_g, const float* go, const float* ol, const float* osp,
                 void* out, hipStream_t st) {
  const int tiles = (s.Lq + 15) / 16;
  hipLaunchKernelGGL((fuse_kernel<T, D>), dim3(tiles), dim3(kFuseThreads), 0, st,
                     reinterpret_cast<const T*>(x), reinterpret_cast<const T*>(w_g), go, ol, osp, s.H, s.Lq,
                     reinterpret_cast<T*>(out));
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_fuse(const hsa_geom* geom, const void* x, const void* w_g, const float* gate_override,
                           const float* o_lin, const float* o_sp, void* out, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!o_lin || !o_sp || !out) return HSA_ERR_NULL_ARG;
  if (x ? !w_g : !gate_override) return HSA_ERR_NULL_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (s.bf16) {
    if (s.d == 128) launch_fuse<bf16_t, 128>(s, x, w_g, gate_override, o_lin, o_sp, out, st);
    else launch_fuse<bf16_t, 64>(s, x, w_g, gate_override, o_lin, o_sp, out, st);
  } else {
    if (s.d == 128) launch_fuse<float, 128>(s, x, w_g, gate_override, o_lin, o_sp, out, st);
    else launch_fuse<float, 64>(s, x, w_g, gate_override, o_lin, o_sp, out, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
