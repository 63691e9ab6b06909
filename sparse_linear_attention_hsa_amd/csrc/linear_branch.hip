// S3 -- linear branch.  WorldAttention paper, section 3.3 "Linear branch"
// (output equation); structured summary, prerequisite "linear attention"
// (Linformer: the sequence axis of K and V is projected to rank r << L).
//   Ktil_h = E_K K_h  [r][d],  Vtil_h = E_V V_h  [r][d],
//   O_lin_h = softmax(Q_h Ktil_h^T / sqrt(d)) Vtil_h.
//
// Kernels:
//  * project: split-K matrix-core product over the sequence axis.  One
//    workgroup (4 waves) computes the full r x d output of one (head, K|V)
//    for one slice of the sequence, so every active K/V element is read from
//    memory exactly once; E (shared by all heads) is re-read from L2/MALL.
//    Contraction over tokens needs tokens contiguous per operand lane: V is
//    already token-contiguous (d-major granules); K tiles are transposed
//    through LDS.  Partials are float32.
//  * reduce : fixed-order sum of the slices, written as Ktil [H][r][d] and
//    Vtil^T [H][d][r] in float32.
//  * attend : per (head, 16-query tile) wave, S^T = Ktil Q^T over all r
//    rows at once (exact softmax, no online rescaling), then O^T = Vtil^T P^T.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kProjThreads = 256;  // 4 waves
constexpr int kMaxRT = 16;         // r-tiles of 16 per workgroup (r <= 256)

// grid = (2*H, splits).  x < H: keys of head x, else values of head x-H.
// Software pipeline: the global loads of step n+1 are in flight while step n
// is multiplied; the transposed K tile is double buffered in LDS (one
// barrier per step).
template <typename T, int D>
__global__ __launch_bounds__(kProjThreads) void lin_project_kernel(
    const T* __restrict__ k_act, const T* __restrict__ v_act, const T* __restrict__ e_k,
    const T* __restrict__ e_v, int H, int L, int r, int steps, int splits, float* __restrict__ partial) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;      // tokens per step
  constexpr int DT = D / 16;
  constexpr int RPW = kMaxRT / 4;    // r-tiles per wave
  constexpr int TSTR = KS + E;       // LDS row stride (elements) of the transposed K tile
  constexpr int KCH = KS * (D / E);  // 16-byte chunks of one K step
  constexpr int KPT = (KCH + kProjThreads - 1) / kProjThreads;
  __shared__ __align__(16) T kt_s[2][D * TSTR];

  const int which = blockIdx.x;
  const bool is_v = which >= H;
  const int h = is_v ? which - H : which;
  const int split = blockIdx.y;
  const int st0 = (int)((long long)steps * split / splits);
  const int st1 = (int)((long long)steps * (split + 1) / splits);
  const T* e = is_v ? e_v : e_k;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int g = lane >> 4, c = lane & 15;
  const int rtiles = (r + 15) / 16;

  f32x4 acc[RPW][DT];
#pragma unroll
  for (int a = 0; a < RPW; ++a)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 aop[RPW], bop[DT], kch[KPT];
  // issue the global loads of one step
  auto load = [&](int stp) {
    const int tok0 = stp * KS;
    const int tk = tok0 + g * E;
#pragma unroll
    for (int a = 0; a < RPW; ++a) {
      const int rr = 16 * (w * RPW + a) + c;
      aop[a] = (rr < r && tk < L) ? ld16(e + (size_t)rr * L + tk) : make_uint4(0, 0, 0, 0);
    }
    if (is_v) {
      // v_act granules [L/16][D][16]: chunk g covers tokens tk .. tk+E-1
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        bop[dt] = tk < L ? ld16(v_act + (((size_t)h * (L / 16) + tk / 16) * D + 16 * dt + c) * 16 + (tk % 16))
                         : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int ci = tid + u * kProjThreads;
        const int tr = ci / (D / E), cc = ci % (D / E);
        kch[u] = (ci < KCH && tok0 + tr < L) ? ld16(k_act + ((size_t)h * L + tok0 + tr) * D + cc * E)
                                             : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // K only: write the loaded rows transposed, kt_s[buf][col][token]
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ci = tid + u * kProjThreads;
      if (ci < KCH) {
        const int tr = ci / (D / E), cc = ci % (D / E);
        float f[E];
        unpack16<T>(kch[u], f);
#pragma unroll
        for (int x = 0; x < E; ++x) kt_s[buf][(cc * E + x) * TSTR + tr] = from_f32<T>(f[x]);
      }
    }
  };

  if (st0 < st1) {
    load(st0);
    if (!is_v) {
      stage(0);
      __syncthreads();
    }
  }
  for (int stp = st0; stp < st1; ++stp) {
    const int buf = (stp - st0) & 1;
    uint4 a_cur[RPW], b_cur[DT];
#pragma unroll
    for (int a = 0; a < RPW; ++a) a_cur[a] = aop[a];
    if (is_v) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) b_cur[dt] = bop[dt];
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) b_cur[dt] = *reinterpret_cast<const uint4*>(&kt_s[buf][(16 * dt + c) * TSTR + g * E]);
    }
    const bool more = stp + 1 < st1;
    if (more) load(stp + 1);
#pragma unroll
    for (int a = 0; a < RPW; ++a) {
      if (w * RPW + a < rtiles) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) Mma<T>::run(acc[a][dt], a_cur[a], b_cur[dt]);
      }
    }
    if (!is_v && more) {
      stage(buf ^ 1);
      __syncthreads();
    }
  }
  // partial[split][which][rt*16 + row][D]; lane holds rows 4g+i, column c of each tile
  float* out = partial + (((size_t)split * 2 * H + which) * (size_t)(rtiles * 16)) * D;
#pragma unroll
  for (int a = 0; a < RPW; ++a) {
    const int rt = w * RPW + a;
    if (rt < rtiles) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(size_t)(16 * rt + 4 * g + i) * D + 16 * dt + c] = acc[a][dt][i];
    }
  }
}

// Sum the split partials in order; write Ktil [H][r][d] and Vtil^T [H][d][r] (float32).
// grid = (2H, ceil(r*D/1024)); each thread sums one float4 column group over the splits.
__global__ __launch_bounds__(256) void lin_reduce_kernel(const float* __restrict__ partial, int H, int D, int r,
                                                         int splits, float* __restrict__ k_proj,
                                                         float* __restrict__ v_proj) {
  const int which = blockIdx.x;
  const bool is_v = which >= H;
  const int h = is_v ? which - H : which;
  const int rpad = (r + 15) / 16 * 16;
  const int e4 = blockIdx.y * 256 + threadIdx.x;  // float4 index inside [r][D]
  if (e4 * 4 >= r * D) return;
  const int rr = (e4 * 4) / D, col = (e4 * 4) % D;
  const size_t stride = (size_t)2 * H * rpad * D;
  const float* p = partial + ((size_t)which * rpad + rr) * D + col;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int sp = 0;
  for (; sp + 4 <= splits; sp += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(p + (size_t)(sp + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
  }
  for (; sp < splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(p + (size_t)sp * stride);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (is_v) {
    float* o = v_proj + ((size_t)h * D + col) * r + rr;
    o[0] = s.x; o[r] = s.y; o[2 * r] = s.z; o[3 * r] = s.w;
  } else {
    *reinterpret_cast<float4*>(k_proj + ((size_t)h * r + rr) * D + col) = s;
  }
}

// A operand of the matrix cores from float32 storage (one chunk of Vec<T>::N
// contraction elements).  For bf16 the value is split into hi = bf16(x) and
// lo = bf16(x - hi): two products carry ~16 mantissa bits, so the projected
// keys keep float32-like precision in the logits even when |Q| is large.
template <typename T> struct F32Operand;
template <> struct F32Operand<float> {
  static constexpr bool kSplit = false;
  __device__ __forceinline__ static void load(const float* p, bool ok, uint4& hi, uint4& lo) {
    hi = ok ? ld16(p) : make_uint4(0, 0, 0, 0);
    lo = make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ static uint4 load_round(const float* p, int n_ok) {
    float f[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) f[x] = x < n_ok ? p[x] : 0.f;
    return pack16<float>(f);
  }
};
template <> struct F32Operand<bf16_t> {
  static constexpr bool kSplit = true;
  __device__ __forceinline__ static void load(const float* p, bool ok, uint4& hi, uint4& lo) {
    float f[8];
    if (ok) {
      const float4 a = reinterpret_cast<const float4*>(p)[0];
      const float4 b = reinterpret_cast<const float4*>(p)[1];
      f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) f[x] = 0.f;
    }
    hi = pack16<bf16_t>(f);
    float fh[8];
    unpack16<bf16_t>(hi, fh);
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] -= fh[x];
    lo = pack16<bf16_t>(f);
  }
  __device__ __forceinline__ static uint4 load_round(const float* p, int n_ok) {
    float f[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = x < n_ok ? p[x] : 0.f;
    return pack16<bf16_t>(f);
  }
};

// One wave per (head, 16-query tile).  S^T tiles cover all (padded) r rows.
// Control flow around the matrix-core products is uniform per wave: rows past
// r load zeros and are masked before the softmax.
template <typename T, int D, int RT>
__global__ __launch_bounds__(256) void lin_attend_kernel(
    const T* __restrict__ q, const float* __restrict__ k_proj, const float* __restrict__ v_proj, int H, int Lq,
    int r, float scale_log2, float* __restrict__ o_lin) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;
  constexpr int DSTEPS = D / KS;
  constexpr int DT = D / 16;
  constexpr int GPS = KS / 16;         // r-tiles per contraction step of the PV product
  const int tid = threadIdx.x, lane = tid % kWave;
  const int g = lane >> 4, c = lane & 15;
  const int tiles_q = (Lq + 15) / 16;
  const int wid = blockIdx.x * 4 + tid / kWave;
  if (wid >= tiles_q * H) return;
  const int h = wid / tiles_q, qt = wid % tiles_q;
  const int qrow = qt * 16 + c;

  uint4 qreg[DSTEPS];
#pragma unroll
  for (int s = 0; s < DSTEPS; ++s)
    qreg[s] = qrow < Lq ? ld16(q + ((size_t)qrow * H + h) * D + (4 * s + g) * E) : make_uint4(0, 0, 0, 0);

  // S^T[r][q]: tile rt row c loads Ktil row 16*(rt - rt%GPS) + perm_row(rt%GPS, c)
  f32x4 sacc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (16 * (rt - rt % GPS) < r) {  // wave-uniform
      const int rr = 16 * (rt - rt % GPS) + perm_row<T>(rt % GPS, c);
      const bool ok = rr < r;
      const float* kp = k_proj + ((size_t)h * r + (ok ? rr : 0)) * D;
#pragma unroll
      for (int s = 0; s < DSTEPS; ++s) {
        uint4 hi, lo;
        F32Operand<T>::load(kp + (4 * s + g) * E, ok, hi, lo);
        Mma<T>::run(sacc[rt], hi, qreg[s]);
        if (F32Operand<T>::kSplit) Mma<T>::run(sacc[rt], lo, qreg[s]);
      }
    }
  }
  // exact softmax over the r rows (rows >= r masked)
  float mx = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * (rt - rt % GPS) + perm_row<T>(rt % GPS, 4 * g + i);
      if (rr >= r) sacc[rt][i] = -INFINITY;
      mx = fmaxf(mx, sacc[rt][i]);
    }
  mx = max4g(mx) * scale_log2;
  float ls = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp2f(sacc[rt][i] * scale_log2 - mx);
      sacc[rt][i] = e;
      ls += e;
    }
  const float inv = 1.f / sum4g(ls);
  // O^T[d][q] = Vtil^T[d][r] P^T[r][q]; step covers r-tiles GPS*st .. +GPS-1
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int stp = 0; stp < RT / GPS; ++stp) {
    if (stp * KS < r) {  // wave-uniform
      const uint4 pb = pack_p<T>(&sacc[stp * GPS]);
      const int r0 = stp * KS + g * E;  // r chunk of this lane group
      const int n_ok = r0 >= r ? 0 : min(E, r - r0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float* vp = v_proj + ((size_t)h * D + 16 * dt + c) * r + (n_ok > 0 ? r0 : 0);
        Mma<T>::run(o[dt], F32Operand<T>::load_round(vp, n_ok), pb);
      }
    }
  }
  if (qrow < Lq) {
    float* dst = o_lin + ((size_t)qrow * H + h) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt) = make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
  }
}

template <typename T, int D>
void launch_linear(const Dims& s, const void* q, const void* k_act, const void* v_act, const void* e_k,
                   const void* e_v, void* k_proj, void* v_proj, float* o_lin, int flags, char* ws,
                   const WsLayout& w, hipStream_t st) {
  const ProjPlan pp = proj_plan(s);
  float* partial = reinterpret_cast<float*>(ws + w.lin_partial);
  if (!(flags & HSA_LIN_REUSE_PROJ)) {
    hipLaunchKernelGGL((lin_project_kernel<T, D>), dim3(2 * s.H, pp.splits), dim3(kProjThreads), 0, st,
                       reinterpret_cast<const T*>(k_act), reinterpret_cast<const T*>(v_act),
                       reinterpret_cast<const T*>(e_k), reinterpret_cast<const T*>(e_v), s.H, s.L, s.r, pp.steps,
                       pp.splits, partial);
    hipLaunchKernelGGL(lin_reduce_kernel, dim3(2 * s.H, (s.r * D / 4 + 255) / 256), dim3(256), 0, st, partial, s.H, D, s.r, pp.splits,
                       reinterpret_cast<float*>(k_proj), reinterpret_cast<float*>(v_proj));
  }
  if (flags & HSA_LIN_PROJ_ONLY) return;
  const int tiles_q = (s.Lq + 15) / 16;
  const int nblk = (tiles_q * s.H + 3) / 4;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
  const int rt = pp.rpad / 16;  // r-tiles covering the padded rank
#define HSA_LIN_CASE(RT_) \
  if (rt <= RT_) { hipLaunchKernelGGL((lin_attend_kernel<T, D, RT_>), dim3(nblk), dim3(256), 0, st, \
      reinterpret_cast<const T*>(q), reinterpret_cast<const float*>(k_proj), reinterpret_cast<const float*>(v_proj), \
      s.H, s.Lq, s.r, scale_log2, o_lin); return; }
  HSA_LIN_CASE(2)
  HSA_LIN_CASE(4)
  HSA_LIN_CASE(8)
  HSA_LIN_CASE(16)
#undef HSA_LIN_CASE
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_linear_branch(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                                    const void* e_k, const void* e_v, void* k_proj, void* v_proj, float* o_lin,
                                    int32_t flags, void* ws, size_t ws_bytes, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (flags & ~(HSA_LIN_REUSE_PROJ | HSA_LIN_PROJ_ONLY)) return HSA_ERR_BAD_PARAM;
  if ((flags & HSA_LIN_REUSE_PROJ) && (flags & HSA_LIN_PROJ_ONLY)) return HSA_ERR_BAD_PARAM;
  if (!k_proj || !v_proj) return HSA_ERR_NULL_ARG;
  if (!(flags & HSA_LIN_REUSE_PROJ) && (!k_act || !v_act || !e_k || !e_v)) return HSA_ERR_NULL_ARG;
  if (!(flags & HSA_LIN_PROJ_ONLY) && (!q || !o_lin)) return HSA_ERR_NULL_ARG;
  const WsLayout w = ws_layout(s, 1);
  if (!(flags & HSA_LIN_REUSE_PROJ) && (!ws || ws_bytes < w.lin_end)) return HSA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  if (s.bf16) {
    if (s.d == 128) launch_linear<bf16_t, 128>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, st);
    else launch_linear<bf16_t, 64>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, st);
  } else {
    if (s.d == 128) launch_linear<float, 128>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, st);
    else launch_linear<float, 64>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
