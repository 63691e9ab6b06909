// S3 -- linear branch.  WorldAttention paper, section 3.3 "Linear branch"
// (output equation); structured summary, prerequisite "linear attention"
// (Linformer: the sequence axis of K and V is projected to rank r << L).
//   Ktil_h = E_K K_h  [r][d],  Vtil_h = E_V V_h  [r][d],
//   O_lin_h = softmax(Q_h Ktil_h^T / sqrt(d)) Vtil_h.
//
// Kernels:
//  * project: split-K matrix-core product over the sequence axis.  One
//    workgroup computes the full r x d outputs of two heads (K or V) for one
//    slice of the sequence, so every active K/V element is read from memory
//    exactly once and each E tile serves two heads.  Contraction over tokens
//    needs tokens contiguous per operand lane: V is already token-contiguous
//    (d-major granules); K tiles are transposed through LDS.  Partials are
//    float32.
//  * reduce : fixed-order sum of the slices, written as Ktil [H][r][d] and
//    Vtil^T [H][d][r] in float32.
//  * attend : 128 queries of one head per workgroup; rank chunks of Ktil and
//    Vtil^T staged in LDS, online softmax over the chunks, O^T = Vtil^T P^T.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// Projection of the sequence axis, split over S slices of the active keys.
// Work item = (slice, K|V, head pair); the two heads of a pair share one E
// tile.  Items run slice-major and each XCD takes a contiguous range of them,
// so the workgroups that need the same E slice sit behind the same L2.
// Workgroup = 8 waves: wave w works on head (w / 4) of the pair and on r-tiles
// 4*(w % 4) .. +3, all D columns (128 float32 accumulators per lane).
// Per stage (2 contraction steps, ST tokens), staged in LDS and double
// buffered:
//  * E tile [256 rows][ST tokens] by direct global->LDS loads; chunk slot
//    swizzled by the row so the operand reads are bank-conflict free;
//  * X^T tiles [D][ST tokens] per head in regions [granule][part][D][16 B]:
//    values arrive that way from the active buffer (direct loads); keys are
//    loaded to registers one stage ahead and written transposed.
constexpr int kProjThreads = 512;  // 8 waves
constexpr int kProjHeads = 2;

__device__ __forceinline__ int eswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <typename T, int D>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_project_kernel(
    const T* __restrict__ k_act, const T* __restrict__ v_act, const T* __restrict__ e_k,
    const T* __restrict__ e_v, int H, int L, int r, int splits, float* __restrict__ partial) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;          // tokens per contraction step
  constexpr int ST = 2 * KS;             // tokens per stage
  constexpr int DT = D / 16;
  constexpr int PV = 16 / E;             // 16-byte parts per granule row
  constexpr int NREG = ST / 16 * PV;     // X^T regions per stage (8)
  constexpr int XBYTES = NREG * D * 16;  // X^T tile bytes per head
  constexpr int EBYTES = 256 * ST * (int)sizeof(T);  // 256 rows x 128 bytes
  constexpr int KCH = ST * (D / E);      // 16-byte key chunks per head per stage
  constexpr int KPT = (kProjHeads * KCH) / kProjThreads;
  __shared__ __align__(1024) unsigned char lds_e[2][EBYTES];
  __shared__ __align__(1024) unsigned char lds_x[2][kProjHeads][XBYTES];

  const int HP = (H + 1) / 2;
  const int n_items = splits * 2 * HP;
  const int item = xcd_remap(blockIdx.x, n_items);
  if (item < 0) return;
  const int split = item / (2 * HP);
  const int kv = (item / HP) % 2;
  const int hp = item % HP;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4, c = lane & 15;
  const int hs = w / 4, rg = w % 4;            // head slot, r-group of this wave
  const int h = hp * 2 + hs;                   // may be == H for an odd head count
  const bool h_ok = h < H;
  const int rtiles = (r + 15) / 16;
  const int nst = (L + ST - 1) / ST;
  const int st0 = (int)((long long)nst * split / splits);
  const int st1 = (int)((long long)nst * (split + 1) / splits);
  const T* e = kv ? e_v : e_k;

  f32x4 acc[4][DT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 kreg[KPT > 0 ? KPT : 1];
  // direct loads of one stage (E for all rows, values for both heads), key rows to registers
  auto issue = [&](int stg, int buf) {
    const int tok0 = stg * ST;
    // E: instruction i covers rows 8i .. 8i+7 (128 bytes each)
    for (int i = w; i < rtiles * 2; i += kProjThreads / kWave) {
      const int row = 8 * i + lane / 8;
      const int chunk = (lane % 8) ^ eswz(row);
      const int tk = tok0 + chunk * E;
      const void* src = (row < r && tk < L) ? (const void*)(e + (size_t)row * L + tk) : (const void*)(kZeroPage + lane);
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds_e[buf] + i * 1024), 16, 0, 0);
    }
    if (kv) {
      // values: region = (granule, part), D/64 instructions per region, per head
#pragma unroll
      for (int ii = 0; ii < (kProjHeads * NREG * D / 64) / (kProjThreads / kWave); ++ii) {
        const int i = ii * (kProjThreads / kWave) + w;
        const int hsl = i / (NREG * D / 64);
        const int rem = i % (NREG * D / 64);
        const int region = rem / (D / 64);
        const int rowv = (rem % (D / 64)) * 64 + lane;
        const int gr = region / PV, part = region % PV;
        const int hh = hp * 2 + hsl;
        const int tk = tok0 + gr * 16;
        const void* src = (hh < H && tk < L)
                              ? (const void*)(v_act + (((size_t)hh * (L / 16) + tk / 16) * D + rowv) * 16 + part * E)
                              : (const void*)(kZeroPage + lane);
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds_x[buf][hsl] + (size_t)region * D * 16 + (rem % (D / 64)) * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int ci = tid + u * kProjThreads;
        const int hsl = ci / KCH, cr = ci % KCH;
        const int tr = cr / (D / E), cc = cr % (D / E);
        const int hh = hp * 2 + hsl;
        kreg[u] = (hh < H && tok0 + tr < L) ? ld16(k_act + ((size_t)hh * L + tok0 + tr) * D + cc * E)
                                           : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // keys only: write the registers of a stage transposed into the X^T regions
  auto stage_keys = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ci = tid + u * kProjThreads;
      const int hsl = ci / KCH, cr = ci % KCH;
      const int tr = cr / (D / E), cc = cr % (D / E);
      const int region = (tr / 16) * PV + (tr % 16) / E;
      unsigned char* base = lds_x[buf][hsl] + (size_t)region * D * 16 + (tr % E) * sizeof(T);
      float f[E];
      unpack16<T>(kreg[u], f);
#pragma unroll
      for (int x = 0; x < E; ++x) *reinterpret_cast<T*>(base + (cc * E + x) * 16) = from_f32<T>(f[x]);
    }
  };

  if (st0 < st1) {
    issue(st0, 0);
    if (!kv) stage_keys(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  for (int stg = st0; stg < st1; ++stg) {
    const int buf = (stg - st0) & 1;
    const bool more = stg + 1 < st1;
    if (more) issue(stg + 1, buf ^ 1);
    if (h_ok && rg * 4 < rtiles) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 bop[DT];
        const unsigned char* xr = lds_x[buf][hs] + (size_t)(ks * 4 + g) * D * 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) bop[dt] = *reinterpret_cast<const uint4*>(xr + (16 * dt + c) * 16);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int row = 16 * (rg * 4 + a) + c;
          const int slot = (ks * 4 + g) ^ eswz(row);
          const uint4 aop = *reinterpret_cast<const uint4*>(lds_e[buf] + row * 128 + slot * 16);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) Mma<T>::run(acc[a][dt], aop, bop[dt]);
        }
      }
    }
    if (more && !kv) stage_keys(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  // partial[split][kv*H + h][rt*16 + row][D]; lane holds rows 4g+i, column c of each tile
  if (!h_ok) return;
  const int which = kv * H + h;
  float* out = partial + (((size_t)split * 2 * H + which) * (size_t)(rtiles * 16)) * D;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int rt = rg * 4 + a;
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

// Attention over the r projected keys.  A workgroup (4 waves x 2 query tiles
// = 128 queries of one head) walks the rank axis in chunks of KS rows; each
// chunk of Ktil (as a bf16 high/low pair, so the logits keep float32-like
// precision) and of Vtil^T (bf16) is staged once in LDS, double buffered, and
// shared by all 128 queries; an online softmax runs over the chunks.  Chunk
// rows past r are zero and masked.
constexpr int kAttQT = 2;                      // query tiles per wave
constexpr int kAttThreads = 256;               // 4 waves
constexpr int kAttRows = 4 * kAttQT * 16;      // queries per workgroup

template <typename T, int D>
__global__ __launch_bounds__(kAttThreads) void lin_attend_kernel(
    const T* __restrict__ q, const float* __restrict__ k_proj, const float* __restrict__ v_proj, int H, int Lq,
    int r, float scale_log2, float* __restrict__ o_lin) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;        // rank rows per chunk (= one PV contraction step)
  constexpr int GPS = KS / 16;         // 16-row tiles per chunk
  constexpr int DSTEPS = D / KS;
  constexpr int DT = D / 16;
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int KSTR = D + E;          // padded LDS rows (elements)
  constexpr int VSTR = KS + E;
  __shared__ __align__(16) T k_hi[2][KS * KSTR];
  __shared__ __align__(16) T k_lo[2][SPLIT ? KS * KSTR : E];
  __shared__ __align__(16) T v_t[2][D * VSTR];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4, c = lane & 15;
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * kAttRows + w * kAttQT * 16;
  const float* kp = k_proj + (size_t)h * r * D;
  const float* vp = v_proj + (size_t)h * D * r;
  const int nchunk = (r + KS - 1) / KS;

  uint4 qreg[kAttQT][DSTEPS];
#pragma unroll
  for (int t = 0; t < kAttQT; ++t) {
    const int qrow = q0 + 16 * t + c;
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s)
      qreg[t][s] = qrow < Lq ? ld16(q + ((size_t)qrow * H + h) * D + (4 * s + g) * E) : make_uint4(0, 0, 0, 0);
  }

  // staging: Ktil rows r0..r0+KS-1 (all D columns) and Vtil^T columns r0..r0+KS-1
  auto stage = [&](int ch, int buf) {
    const int r0 = ch * KS;
    for (int e = tid; e < KS * (D / 4); e += kAttThreads) {
      const int rr = e / (D / 4), c4 = e % (D / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + rr < r) v = reinterpret_cast<const float4*>(kp + (size_t)(r0 + rr) * D)[c4];
      const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const T hi = from_f32<T>(f[x]);
        k_hi[buf][rr * KSTR + 4 * c4 + x] = hi;
        if (SPLIT) k_lo[buf][rr * KSTR + 4 * c4 + x] = from_f32<T>(f[x] - to_f32<T>(hi));
      }
    }
    for (int e = tid; e < D * KS; e += kAttThreads) {
      const int dr = e / KS, rr = e % KS;
      const float v = r0 + rr < r ? vp[(size_t)dr * r + r0 + rr] : 0.f;
      v_t[buf][dr * VSTR + rr] = from_f32<T>(v);
    }
  };

  f32x4 o[kAttQT][DT];
  float m_run[kAttQT], l_run[kAttQT];
#pragma unroll
  for (int t = 0; t < kAttQT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  stage(0, 0);
  __syncthreads();
  for (int ch = 0; ch < nchunk; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunk) stage(ch + 1, buf ^ 1);
    f32x4 sacc[kAttQT][GPS];
#pragma unroll
    for (int t = 0; t < kAttQT; ++t)
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt) sacc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < GPS; ++kt) {
      const int rho = perm_row<T>(kt, c);
#pragma unroll
      for (int s = 0; s < DSTEPS; ++s) {
        const uint4 ah = *reinterpret_cast<const uint4*>(&k_hi[buf][rho * KSTR + (4 * s + g) * E]);
#pragma unroll
        for (int t = 0; t < kAttQT; ++t) Mma<T>::run(sacc[t][kt], ah, qreg[t][s]);
        if (SPLIT) {
          const uint4 al = *reinterpret_cast<const uint4*>(&k_lo[buf][rho * KSTR + (4 * s + g) * E]);
#pragma unroll
          for (int t = 0; t < kAttQT; ++t) Mma<T>::run(sacc[t][kt], al, qreg[t][s]);
        }
      }
    }
    const bool ragged = (ch + 1) * KS > r;  // uniform
    uint4 pk[kAttQT];
#pragma unroll
    for (int t = 0; t < kAttQT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (ragged && ch * KS + perm_row<T>(kt, 4 * g + i) >= r) sacc[t][kt][i] = -INFINITY;
          mx = fmaxf(mx, sacc[t][kt][i]);
        }
      mx = max4g(mx) * scale_log2;
      const float m_new = fmaxf(m_run[t], mx);
      const float alpha = fast_exp2(m_run[t] - m_new);
      float ls = 0.f;
      f32x4 p[GPS];
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(sacc[t][kt][i], scale_log2, -m_new));
          p[kt][i] = e;
          ls += e;
        }
      l_run[t] = l_run[t] * alpha + ls;
      m_run[t] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
      pk[t] = pack_p<T>(p);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 a = *reinterpret_cast<const uint4*>(&v_t[buf][(16 * dt + c) * VSTR + g * E]);
#pragma unroll
      for (int t = 0; t < kAttQT; ++t) Mma<T>::run(o[t][dt], a, pk[t]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < kAttQT; ++t) {
    const int qrow = q0 + 16 * t + c;
    if (qrow < Lq) {
      const float inv = 1.f / sum4g(l_run[t]);
      float* dst = o_lin + ((size_t)qrow * H + h) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(dst + 16 * dt) =
            make_float4(o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv, o[t][dt][3] * inv);
    }
  }
}

template <typename T, int D>
void launch_linear(const Dims& s, const void* q, const void* k_act, const void* v_act, const void* e_k,
                   const void* e_v, void* k_proj, void* v_proj, float* o_lin, int flags, char* ws,
                   const WsLayout& w, hipStream_t st) {
  const ProjPlan pp = proj_plan(s);
  float* partial = reinterpret_cast<float*>(ws + w.lin_partial);
  if (!(flags & HSA_LIN_REUSE_PROJ)) {
    const int n_items = pp.splits * 2 * ((s.H + 1) / 2);
    hipLaunchKernelGGL((lin_project_kernel<T, D>), dim3((n_items + 7) / 8 * 8), dim3(kProjThreads), 0, st,
                       reinterpret_cast<const T*>(k_act), reinterpret_cast<const T*>(v_act),
                       reinterpret_cast<const T*>(e_k), reinterpret_cast<const T*>(e_v), s.H, s.L, s.r, pp.splits,
                       partial);
    hipLaunchKernelGGL(lin_reduce_kernel, dim3(2 * s.H, (s.r * D / 4 + 255) / 256), dim3(256), 0, st, partial, s.H, D, s.r, pp.splits,
                       reinterpret_cast<float*>(k_proj), reinterpret_cast<float*>(v_proj));
  }
  if (flags & HSA_LIN_PROJ_ONLY) return;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
  hipLaunchKernelGGL((lin_attend_kernel<T, D>), dim3((s.Lq + kAttRows - 1) / kAttRows, s.H), dim3(kAttThreads), 0, st,
                     reinterpret_cast<const T*>(q), reinterpret_cast<const float*>(k_proj),
                     reinterpret_cast<const float*>(v_proj), s.H, s.Lq, s.r, scale_log2, o_lin);
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
