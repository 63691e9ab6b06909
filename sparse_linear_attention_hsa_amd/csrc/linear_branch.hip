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
// 32-bit LDS address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// N transposing 64-bit LDS reads (ds_read_b64_tr_b16) issued back to back,
// with the wait for all of them inside the same asm statement, so the
// outputs are complete when the statement ends.
template <int N> __device__ __forceinline__ void tr_read_b16(const uint32_t* addr, uint2* out);
template <> __device__ __forceinline__ void tr_read_b16<16>(const uint32_t* a, uint2* o) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %17\n ds_read_b64_tr_b16 %2, %18\n"
      "ds_read_b64_tr_b16 %3, %19\n ds_read_b64_tr_b16 %4, %20\n ds_read_b64_tr_b16 %5, %21\n"
      "ds_read_b64_tr_b16 %6, %22\n ds_read_b64_tr_b16 %7, %23\n ds_read_b64_tr_b16 %8, %24\n"
      "ds_read_b64_tr_b16 %9, %25\n ds_read_b64_tr_b16 %10, %26\n ds_read_b64_tr_b16 %11, %27\n"
      "ds_read_b64_tr_b16 %12, %28\n ds_read_b64_tr_b16 %13, %29\n ds_read_b64_tr_b16 %14, %30\n"
      "ds_read_b64_tr_b16 %15, %31\n s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]),
        "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
      : "memory");
}
template <> __device__ __forceinline__ void tr_read_b16<8>(const uint32_t* a, uint2* o) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %9\n ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n ds_read_b64_tr_b16 %4, %12\n ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n ds_read_b64_tr_b16 %7, %15\n s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Projection of the sequence axis, split over S slices of the active keys.
// Work item = (slice, K|V, head pair); the two heads of a pair share one E
// tile.  Items run slice-major and each XCD takes a contiguous range of them,
// so the workgroups that need the same E slice sit behind the same L2.
// Workgroup = 8 waves: wave w works on head (w / 4) of the pair and on r-tiles
// 4*(w % 4) .. +3, all D columns (128 float32 accumulators per lane).
// One stage = two contraction steps (ST tokens), staged in LDS by direct
// global->LDS loads, double buffered.  The main loop is unrolled by two so
// that every LDS operand read names a fixed buffer: the compiler can then see
// that the loads in flight (other buffer) do not alias the reads, and does not
// stall the reads on them.
//  * E tile [256 rows][ST tokens] (128-byte rows, chunk slot swizzled by row);
//  * values: X^T tile [D][ST tokens] in regions [granule][part][D][16 B], as
//    they arrive from the active buffer;
//  * keys: rows [ST tokens][D], chunk slot swizzled by the token's lane group,
//    read back transposed (ds_read_b64_tr_b16 for bf16).
constexpr int kProjThreads = 512;  // 8 waves
constexpr int kProjHeads = 2;

template <typename T, int D>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_project_kernel(
    const T* __restrict__ k_act, const T* __restrict__ v_act, const T* __restrict__ e_k,
    const T* __restrict__ e_v, int H, int L, int r, int splits, float* __restrict__ partial) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;                      // tokens per contraction step
  constexpr int ST = 2 * KS;                         // tokens per stage
  constexpr int DT = D / 16;
  constexpr int PV = 16 / E;                         // 16-byte parts per granule row
  constexpr int NW = kProjThreads / kWave;
  constexpr int EROW = ST * (int)sizeof(T);          // 128 bytes
  constexpr int EBYTES = 256 * EROW;                 // 32 KB
  constexpr int XBYTES = ST * D * (int)sizeof(T);    // per head
  constexpr int EINST = EBYTES / 1024;
  constexpr int XINST = kProjHeads * XBYTES / 1024;
  constexpr int KROWS = 1024 / (D * (int)sizeof(T)); // key rows per 1 KB instruction
  // one LDS object per buffer, so alias analysis can tell the buffer being
  // read from the one being filled
  __shared__ __align__(1024) unsigned char lds_e0[EBYTES];
  __shared__ __align__(1024) unsigned char lds_e1[EBYTES];
  __shared__ __align__(1024) unsigned char lds_x0[kProjHeads * XBYTES];
  __shared__ __align__(1024) unsigned char lds_x1[kProjHeads * XBYTES];

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
  // E rows: 16-byte chunk slot XOR eswz(row): the 16 rows read together by a
  // lane group land on distinct banks
  auto eswz = [](int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); };
  // keys: 16-byte chunk slot XOR kslot(token); for bf16 this moves whole
  // 32-byte column groups, so the 16 rows of one transposing read spread over
  // the banks.  (For f32 the XOR only separates the gathered lane groups.)
  auto kslot = [](int tr) {
    if (sizeof(T) == 2) return 2 * (((tr & 3) | (((tr >> 3) & 1) << 2)) & (D / 16 - 1));
    return ((tr % KS) / E) * PV;
  };

  f32x4 acc[4][DT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int stg, unsigned char* le, unsigned char* lx) {
    const int tok0 = stg * ST;
#pragma unroll
    for (int ii = 0; ii < EINST / NW; ++ii) {
      const int i = ii * NW + w;
      const int row = (1024 / EROW) * i + lane / (EROW / 16);
      const int chunk = (lane % (EROW / 16)) ^ eswz(row);
      const int tk = tok0 + chunk * E;
      const void* src = (row < r && tk < L) ? (const void*)(e + (size_t)row * L + tk) : (const void*)(kZeroPage + lane);
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(le + i * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int ii = 0; ii < XINST / NW; ++ii) {
      const int i = ii * NW + w;
      const int hsl = i / (XBYTES / 1024);
      const int j = i % (XBYTES / 1024);            // 1 KB piece of this head's tile
      const int hh = hp * 2 + hsl;
      const void* src;
      if (kv) {
        // regions [granule][part][D rows][16 B]; piece j = region j/(D/64), rows (j%(D/64))*64 + lane
        const int region = j / (D / 64);
        const int rowv = (j % (D / 64)) * 64 + lane;
        const int gr = region / PV, part = region % PV;
        const int tk = tok0 + gr * 16;
        src = (hh < H && tk < L)
                  ? (const void*)(v_act + (((size_t)hh * (L / 16) + tk / 16) * D + rowv) * 16 + part * E)
                  : (const void*)(kZeroPage + lane);
      } else {
        const int tr = j * KROWS + lane / (D / E);
        const int chunk = (lane % (D / E)) ^ kslot(tr);
        src = (hh < H && tok0 + tr < L) ? (const void*)(k_act + ((size_t)hh * L + tok0 + tr) * D + chunk * E)
                                        : (const void*)(kZeroPage + lane);
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lx + hsl * XBYTES + j * 1024), 16, 0, 0);
    }
  };

  // A operands of one contraction step: E rows of this wave's four r-tiles
  auto load_a = [&](const unsigned char* le, int ks, uint4* aop) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = 16 * (rg * 4 + a) + c;
      aop[a] = *reinterpret_cast<const uint4*>(le + row * EROW + (((ks * 4 + g) ^ eswz(row)) * 16));
    }
  };
  auto compute_v = [&](const unsigned char* le, const unsigned char* lx) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 aop[4];
      load_a(le, ks, aop);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint4 bop = *reinterpret_cast<const uint4*>(lx + (size_t)(ks * 4 + g) * D * 16 + (16 * dt + c) * 16);
#pragma unroll
        for (int a = 0; a < 4; ++a) Mma<T>::run(acc[a][dt], aop[a], bop);
      }
    }
  };
  auto compute_k = [&](const unsigned char* le, const unsigned char* lx) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 aop[4];
      load_a(le, ks, aop);
      if constexpr (sizeof(T) == 2) {
        // transposing LDS reads: lane j of a 16-lane group reads 4 columns
        // 16*dt + 4*(j%4) of token row T0 + j/4; lane c then holds column
        // 16*dt + c of tokens T0 .. T0+3.  Two reads cover the 8 tokens of
        // lane group g.  Four d-tiles per batch of reads.
        const int jc = c & 3, jr = c >> 2;
#pragma unroll
        for (int half = 0; half < DT / 4; ++half) {
          uint32_t addr[8];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int dt = 4 * half + q;
              const int tr = ks * KS + g * 8 + hh * 4 + jr;
              const int chunk = 2 * dt + (jc >> 1);
              addr[2 * q + hh] = lds_addr(lx + (size_t)tr * D * 2 + ((chunk ^ kslot(tr)) * 16) + 8 * (jc & 1));
            }
          uint4 bop[4];
          tr_read_b16<8>(addr, reinterpret_cast<uint2*>(bop));
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int a = 0; a < 4; ++a) Mma<T>::run(acc[a][4 * half + q], aop[a], bop[q]);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int col = 16 * dt + c;
          T v[E];
#pragma unroll
          for (int x = 0; x < E; ++x) {
            const int tr = ks * KS + g * E + x;
            v[x] = *reinterpret_cast<const T*>(lx + (size_t)tr * D * sizeof(T) +
                                               (((col / E) ^ kslot(tr)) * 16) + (col % E) * sizeof(T));
          }
          const uint4 bop = *reinterpret_cast<const uint4*>(v);
#pragma unroll
          for (int a = 0; a < 4; ++a) Mma<T>::run(acc[a][dt], aop[a], bop);
        }
      }
    }
  };
  const bool active = h_ok && rg * 4 < rtiles;  // wave-uniform
  // double-buffered main loop, unrolled by two so every LDS buffer is a fixed object
  auto run = [&](auto&& compute) {
    if (st0 < st1) {
      issue(st0, lds_e0, lds_x0);
      __syncthreads();
    }
    for (int stg = st0; stg < st1; stg += 2) {
      if (stg + 1 < st1) issue(stg + 1, lds_e1, lds_x1);
      if (active) compute(lds_e0, lds_x0 + hs * XBYTES);
      __syncthreads();
      if (stg + 1 >= st1) break;
      if (stg + 2 < st1) issue(stg + 2, lds_e0, lds_x0);
      if (active) compute(lds_e1, lds_x1 + hs * XBYTES);
      __syncthreads();
    }
  };
  if (kv) run(compute_v);
  else run(compute_k);

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
