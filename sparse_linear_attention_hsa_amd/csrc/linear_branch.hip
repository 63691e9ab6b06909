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

// 32-bit LDS address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// N transposing 64-bit LDS reads (ds_read_b64_tr_b16) issued back to back,
// with the wait for all of them inside the same asm statement, so the outputs
// are complete when the statement ends.  (The addresses here are 32-bit LDS
// offsets built by integer arithmetic; the compiler's own form of this read,
// given such an address, cannot tell it from the direct-to-LDS loads in
// flight and waits for all of them first.)
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
// One stage = one contraction step (KS tokens), staged in LDS by direct
// global->LDS loads into a ring of kProjRing slots: while one stage is
// multiplied, the loads of the next kProjRing-1 stages are in flight.  Every
// slot is its own LDS object and the main loop is unrolled over the ring, so
// each operand read names a fixed slot: the compiler can then see that the
// loads in flight (other slots) do not alias the reads and does not stall the
// reads on them.  The waits count the loads still allowed in flight
// (ring_barrier) instead of draining them all at each barrier.
//  * E tile [256 rows][KS tokens] (64-byte rows, chunk slot swizzled by row);
//  * values: X^T tile [D][KS tokens] in regions [granule][part][D][16 B], as
//    they arrive from the active buffer;
//  * keys: rows [KS tokens][D], chunk slot swizzled by the token's lane group,
//    read back transposed (ds_read_b64_tr_b16 for bf16).
constexpr int kProjThreads = 512;  // 8 waves
constexpr int kProjHeads = 2;
constexpr int kProjRing = 4;

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_project_kernel(
    const T* __restrict__ k_act, const T* __restrict__ v_act, const T* __restrict__ e_k,
    const T* __restrict__ e_v, int H, int L, int r, int splits, int t_begin, int t_end, float* __restrict__ partial,
    PagedKV<PAGED> pg) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;                      // tokens per stage (one contraction step)
  constexpr int DT = D / 16;
  constexpr int PV = 16 / E;                         // 16-byte parts per granule row
  constexpr int NW = kProjThreads / kWave;
  constexpr int EROW = KS * (int)sizeof(T);          // 64 bytes
  constexpr int EBYTES = 256 * EROW;                 // 16 KB
  constexpr int XBYTES = KS * D * (int)sizeof(T);    // per head
  constexpr int EINST = EBYTES / 1024;
  constexpr int XINST = kProjHeads * XBYTES / 1024;
  constexpr int KROWS = 1024 / (D * (int)sizeof(T)); // key rows per 1 KB instruction
  constexpr int PER = EINST / NW + XINST / NW;       // loads per wave per stage
  static_assert(EROW == 64 && EINST % NW == 0 && XINST % NW == 0, "stage tiling");
  static_assert((kProjRing - 2) * PER < 64, "vmcnt range");
  // one LDS object per slot (see above)
  __shared__ __align__(1024) unsigned char lds_e0[EBYTES];
  __shared__ __align__(1024) unsigned char lds_e1[EBYTES];
  __shared__ __align__(1024) unsigned char lds_e2[EBYTES];
  __shared__ __align__(1024) unsigned char lds_e3[EBYTES];
  __shared__ __align__(1024) unsigned char lds_x0[kProjHeads * XBYTES];
  __shared__ __align__(1024) unsigned char lds_x1[kProjHeads * XBYTES];
  __shared__ __align__(1024) unsigned char lds_x2[kProjHeads * XBYTES];
  __shared__ __align__(1024) unsigned char lds_x3[kProjHeads * XBYTES];

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
  // the contraction runs over active tokens [t_begin, t_end) (row strides stay L)
  const int nst = (t_end - t_begin + KS - 1) / KS;
  const int st0 = (int)((long long)nst * split / splits);
  const int st1 = (int)((long long)nst * (split + 1) / splits);
  const T* e = kv ? e_v : e_k;
  // E rows (four 16-byte chunks): chunk slot XOR ((row >> 2) & 3); the 16
  // rows one lane group reads at one chunk index then cover 16 distinct
  // 16-byte bank groups
  auto eswz = [](int row) { return (row >> 2) & 3; };
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

  // exactly PER loads per wave (tails read the zero page), so the waits can count them
  auto issue = [&](int stg, unsigned char* le, unsigned char* lx) {
    const int tok0 = t_begin + stg * KS;
    // paged: the stage's KS tokens lie in at most two pages (16-token
    // granules never straddle one); tokens from bnd on are in the second
    int bnd = 0, first = 0;
    const T* kpage[2] = {nullptr, nullptr};
    const T* vpage[2] = {nullptr, nullptr};
    if constexpr (PAGED) {
      const int kp = (L + pg.Lp - 1) / pg.Lp;  // pages of the active keys (the chunk's last one may be partial)
      const int p0 = tok0 / pg.Lp, p1 = min(p0 + 1, kp - 1);
      first = p0 * pg.Lp;
      bnd = first + pg.Lp;
      int pa = pg.sel[p0], pb = pg.sel[p1];
      pa = pa < 0 ? 0 : (pa >= pg.n_pages ? pg.n_pages - 1 : pa);
      pb = pb < 0 ? 0 : (pb >= pg.n_pages ? pg.n_pages - 1 : pb);
      kpage[0] = reinterpret_cast<const T*>(pg.kpage(pa));
      kpage[1] = reinterpret_cast<const T*>(pg.kpage(pb));
      vpage[0] = reinterpret_cast<const T*>(pg.vpage(pa));
      vpage[1] = reinterpret_cast<const T*>(pg.vpage(pb));
    }
#pragma unroll
    for (int ii = 0; ii < EINST / NW; ++ii) {
      const int i = ii * NW + w;
      const int row = (1024 / EROW) * i + lane / (EROW / 16);
      const int chunk = (lane % (EROW / 16)) ^ eswz(row);
      const int tk = tok0 + chunk * E;
      const void* src = (row < r && tk < t_end) ? (const void*)(e + (size_t)row * L + tk) : (const void*)(kZeroPage + lane);
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
        if constexpr (PAGED) {
          const bool second = tk >= bnd;
          const int lt = tk - (second ? bnd : first);
          const T* vp = second ? vpage[1] : vpage[0];  // (NULL: a page of a device table without one)
          src = (hh < H && tk < t_end && vp != nullptr)
                    ? (const void*)(vp + (((size_t)hh * (pg.Lp / 16) + lt / 16) * D + rowv) * 16 + part * E)
                    : (const void*)(kZeroPage + lane);
        } else {
          src = (hh < H && tk < t_end)
                    ? (const void*)(v_act + (((size_t)hh * (L / 16) + tk / 16) * D + rowv) * 16 + part * E)
                    : (const void*)(kZeroPage + lane);
        }
      } else {
        const int tr = j * KROWS + lane / (D / E);
        const int chunk = (lane % (D / E)) ^ kslot(tr);
        if constexpr (PAGED) {
          const int tk = tok0 + tr;
          const bool second = tk >= bnd;
          const int lt = tk - (second ? bnd : first);
          const T* kp = second ? kpage[1] : kpage[0];
          src = (hh < H && tk < t_end && kp != nullptr)
                    ? (const void*)(kp + ((size_t)hh * pg.Lp + lt) * D + chunk * E)
                    : (const void*)(kZeroPage + lane);
        } else {
          src = (hh < H && tok0 + tr < t_end) ? (const void*)(k_act + ((size_t)hh * L + tok0 + tr) * D + chunk * E)
                                          : (const void*)(kZeroPage + lane);
        }
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lx + hsl * XBYTES + j * 1024), 16, 0, 0);
    }
  };

  // A operands: E rows of this wave's four r-tiles at chunk g
  auto load_a = [&](const unsigned char* le, uint4* aop) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = 16 * (rg * 4 + a) + c;
      aop[a] = *reinterpret_cast<const uint4*>(le + row * EROW + ((g ^ eswz(row)) * 16));
    }
  };
  // Every operand of a stage is read before its products, so one wait covers
  // the LDS latency of the stage instead of one wait per pair of d-tiles.
  auto mma_all = [&](const uint4* aop, const uint4* bop) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) Mma<T>::run(acc[a][dt], aop[a], bop[dt]);
  };
  auto compute_v = [&](const unsigned char* le, const unsigned char* lxs) {
    const unsigned char* lx = lxs + hs * XBYTES;
    uint4 aop[4], bop[DT];
    load_a(le, aop);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      bop[dt] = *reinterpret_cast<const uint4*>(lx + (size_t)g * D * 16 + (16 * dt + c) * 16);
    mma_all(aop, bop);
    // keep the reads ahead of the products (the scheduler would otherwise
    // sink each read to its first use)
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + DT, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * DT, 0);
  };
  auto compute_k = [&](const unsigned char* le, const unsigned char* lxs) {
    const unsigned char* lx = lxs + hs * XBYTES;
    uint4 aop[4], bop[DT];
    load_a(le, aop);
    if constexpr (sizeof(T) == 2) {
      // transposing LDS reads: lane j of a 16-lane group reads 4 columns
      // 16*dt + 4*(j%4) of token row T0 + j/4; lane c then holds column
      // 16*dt + c of tokens T0 .. T0+3.  Two reads cover the 8 tokens of
      // lane group g.
      const int jc = c & 3, jr = c >> 2;
      // the slot base goes through an empty asm so that the 2*DT addresses
      // are formed here from lane offsets, not kept live per slot
      uint32_t xb = lds_addr(lx);
      asm volatile("" : "+v"(xb));
      uint32_t addr[2 * DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int tr = g * 8 + hh * 4 + jr;
          const int chunk = 2 * dt + (jc >> 1);
          addr[2 * dt + hh] = xb + (uint32_t)(tr * D * 2 + ((chunk ^ kslot(tr)) * 16) + 8 * (jc & 1));
        }
      tr_read_b16<2 * DT>(addr, reinterpret_cast<uint2*>(bop));
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = 16 * dt + c;
        T v[E];
#pragma unroll
        for (int x = 0; x < E; ++x) {
          const int tr = g * E + x;
          v[x] = *reinterpret_cast<const T*>(lx + (size_t)tr * D * sizeof(T) +
                                             (((col / E) ^ kslot(tr)) * 16) + (col % E) * sizeof(T));
        }
        bop[dt] = *reinterpret_cast<const uint4*>(v);
      }
    }
    mma_all(aop, bop);
  };
  const bool active = h_ok && rg * 4 < rtiles;  // wave-uniform
  // One ring step: stage i lands (the stages after it, up to two, may stay in
  // flight), every wave is done with the slot of stage i-1, which then takes
  // stage i+3, and stage i is multiplied.
  auto step = [&](int i, const unsigned char* ce, const unsigned char* cx, unsigned char* re, unsigned char* rx,
                  auto&& compute) {
    const int later = st1 - 1 - i;  // stages already issued after i: min(later, 2)
    if (later >= 2) ring_barrier<2 * PER>();
    else if (later == 1) ring_barrier<PER>();
    else ring_barrier<0>();
    if (i + 3 < st1) issue(i + 3, re, rx);
    if (active) compute(ce, cx);
  };
  auto run = [&](auto&& compute) {
    if (st0 < st1) issue(st0, lds_e0, lds_x0);
    if (st0 + 1 < st1) issue(st0 + 1, lds_e1, lds_x1);
    if (st0 + 2 < st1) issue(st0 + 2, lds_e2, lds_x2);
    for (int i = st0; i < st1; i += kProjRing) {
      step(i, lds_e0, lds_x0, lds_e3, lds_x3, compute);
      if (i + 1 < st1) step(i + 1, lds_e1, lds_x1, lds_e0, lds_x0, compute);
      if (i + 2 < st1) step(i + 2, lds_e2, lds_x2, lds_e1, lds_x1, compute);
      if (i + 3 < st1) step(i + 3, lds_e3, lds_x3, lds_e2, lds_x2, compute);
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

// Sum the split partials in order; write Ktil [H][r][d] and Vtil^T [H][d][r]
// (float32), each added to a given base of the same layout when there is one
// (the history's projections, to which the chunk's are added).
// grid = (2H, ceil(r*D/1024)); each thread sums one float4 column group over the splits.
__global__ __launch_bounds__(256) void lin_reduce_kernel(const float* __restrict__ partial, int H, int D, int r,
                                                         int splits, const float* __restrict__ base_k,
                                                         const float* __restrict__ base_v, float* __restrict__ k_proj,
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
    const size_t o0 = ((size_t)h * D + col) * r + rr;
    if (base_v) {
      s.x += base_v[o0]; s.y += base_v[o0 + r]; s.z += base_v[o0 + 2 * r]; s.w += base_v[o0 + 3 * r];
    }
    float* o = v_proj + o0;
    o[0] = s.x; o[r] = s.y; o[2 * r] = s.z; o[3 * r] = s.w;
  } else {
    const size_t o0 = ((size_t)h * r + rr) * D + col;
    if (base_k) {
      const float4 b = *reinterpret_cast<const float4*>(base_k + o0);
      s.x += b.x; s.y += b.y; s.z += b.z; s.w += b.w;
    }
    *reinterpret_cast<float4*>(k_proj + o0) = s;
  }
}

// Operands of the attention over the rank axis, prepared once per call from
// the float32 projections: Ktil as element-type rows [H][rpad][D] and Vtil^T
// as [H][D][rpad], for bf16 each as a high part plus the bf16 rounding of the
// remainder, so the paired products keep float32-like logits and values;
// rows and columns past r are zero.  grid (ceil(rpad*D/256), H, 2): z = 0
// Ktil, 1 Vtil^T.
template <typename T>
__global__ __launch_bounds__(256) void lin_prep_kernel(const float* __restrict__ k_proj,
                                                       const float* __restrict__ v_proj, int D, int r, int rpad,
                                                       T* __restrict__ khi, T* __restrict__ klo, T* __restrict__ vt,
                                                       T* __restrict__ vlo) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= rpad * D) return;
  if (blockIdx.z == 0) {
    const int rr = e / D, col = e % D;
    const float v = rr < r ? k_proj[((size_t)h * r + rr) * D + col] : 0.f;
    const T hi = from_f32<T>(v);
    khi[(size_t)h * rpad * D + e] = hi;
    if (sizeof(T) == 2) klo[(size_t)h * rpad * D + e] = from_f32<T>(v - to_f32<T>(hi));
  } else {
    const int col = e / rpad, rr = e % rpad;
    const float v = rr < r ? v_proj[((size_t)h * D + col) * r + rr] : 0.f;
    const T hi = from_f32<T>(v);
    vt[(size_t)h * D * rpad + e] = hi;
    if (sizeof(T) == 2) vlo[(size_t)h * D * rpad + e] = from_f32<T>(v - to_f32<T>(hi));
  }
}

// Attention over the r projected keys.  A workgroup (8 waves) takes a run of
// 32-query units of one head, eight at a time (one per wave: a pass).  The
// rank axis is streamed in chunks of KS ranks: each chunk's Ktil rows and
// Vtil^T columns (for bf16 both high and low parts) are staged in LDS by
// direct loads, in a ring of four slots three chunks ahead, and all eight
// waves read them from there, so a chunk crosses the L2 once per pass
// instead of once per wave.  Per chunk every wave computes S^T = Ktil Q^T
// (ranks on the rows, one query per accumulator column), an online softmax
// with lazy rescale, and O^T += Vtil^T P^T.  For bf16 the weights are
// rounded to bf16 for the product, and the denominator is the product of an
// all-ones tile with the same packed weights, so numerator and denominator
// use identical weights.  Chunk rows past r are masked.
constexpr int kAttWaves = 8;
constexpr int kAttThreads = kAttWaves * kWave;
constexpr int kAttUnit = 32;  // queries per unit: two 16-row tiles share every Ktil operand read
constexpr int kAttRing = 4;

// V^T chunk rows are 64 bytes (KS ranks): 16-byte slot = chunk ^ vswz(row),
// so the 16 rows one lane group reads at one chunk index use distinct banks.
__device__ __forceinline__ int vswz(int row) { return (row >> 2) & 3; }

template <typename T, int D>
__global__ __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_attend_kernel(
    const T* __restrict__ q, const T* __restrict__ khi, const T* __restrict__ klo, const T* __restrict__ vt,
    const T* __restrict__ vlo, int H, int Lq, int r, int rpad, int units_per_wg, float scale_log2,
    float* __restrict__ o_lin) {
  constexpr int E = Vec<T>::N;
  constexpr int KS = Mma<T>::K;        // ranks per chunk (= one PV contraction step)
  constexpr int GPS = KS / 16;         // 16-row tiles per chunk
  constexpr int CPR = D / E;           // 16-byte chunks per Ktil row
  constexpr int DSTEPS = D / KS;
  constexpr int DT = D / 16;
  constexpr int QT = kAttUnit / 16;
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int NPART = SPLIT ? 2 : 1;
  constexpr int KROWB = D * (int)sizeof(T);
  constexpr int KBYTES = KS * KROWB;   // one part of a chunk's Ktil rows
  constexpr int VROWB = KS * (int)sizeof(T);
  constexpr int VBYTES = D * VROWB;    // one part of a chunk's Vtil^T columns
  constexpr int KRPI = 1024 / KROWB;   // Ktil rows per direct-load instruction
  constexpr int VRPI = 1024 / VROWB;   // Vtil^T rows per instruction
  constexpr int VCPR = VROWB / 16;     // 16-byte chunks per Vtil^T row
  constexpr int NINST = NPART * (KBYTES + VBYTES) / 1024;
  constexpr int PER = NINST / kAttWaves;  // direct loads per wave per chunk
  constexpr int STAGE = NPART * (KBYTES + VBYTES);
  static_assert(VROWB == 64 && VCPR == 4, "V^T chunk rows of 64 bytes");
  static_assert(NINST % kAttWaves == 0 && PER < 64, "stage tiling");
  // one LDS object per ring slot, so every operand read names a fixed slot
  // and the compiler does not make it wait for the loads into the others
  __shared__ __align__(1024) unsigned char lds0[STAGE], lds1[STAGE], lds2[STAGE], lds3[STAGE];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4, c = lane & 15;
  const int h = blockIdx.y;
  const int nchunk = rpad / KS;
  const int units = (Lq + kAttUnit - 1) / kAttUnit;
  const int u_begin = blockIdx.x * units_per_wg;
  const int u_end = min(units, u_begin + units_per_wg);
  if (u_begin >= u_end) return;  // uniform over the workgroup
  const int passes = (u_end - u_begin + kAttWaves - 1) / kAttWaves;
  const int nst = passes * nchunk;
  const T* kh = khi + (size_t)h * rpad * D;
  const T* kl = klo + (size_t)h * rpad * D;
  const T* vh = vt + (size_t)h * D * rpad;
  const T* vl = vlo + (size_t)h * D * rpad;

  // chunk (stage % nchunk) into one slot: [Ktil hi][Ktil lo][Vt hi][Vt lo]
  auto issue = [&](int stage, unsigned char* slot) {
    const int ch = stage % nchunk;
#pragma unroll
    for (int ii = 0; ii < PER; ++ii) {
      const int i = ii * kAttWaves + w;  // instruction index in the stage
      const void* src;
      if (i < NPART * KBYTES / 1024) {
        const int part = i / (KBYTES / 1024), k = i % (KBYTES / 1024);
        const int row = k * KRPI + lane / CPR;  // row inside the chunk
        const int chunk = (lane % CPR) ^ kswz<T>(row, CPR);
        src = (part ? kl : kh) + (size_t)(ch * KS + row) * D + chunk * E;
      } else {
        const int iv = i - NPART * KBYTES / 1024;
        const int part = iv / (VBYTES / 1024), k = iv % (VBYTES / 1024);
        const int row = k * VRPI + lane / VCPR;  // d row
        const int chunk = (lane % VCPR) ^ vswz(row);
        src = (part ? vl : vh) + (size_t)row * rpad + ch * KS + chunk * E;
      }
      load_lds16(src, slot + i * 1024);
    }
  };

  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0 pairs
  uint4 qreg[QT][DSTEPS];
  f32x4 o[QT][DT];
  f32x4 lacc[QT];  // bf16: denominators from the ones tile
  float m_run[QT], l_run[QT];

  // one chunk of ranks against this wave's unit
  auto compute = [&](int ch, const unsigned char* slot) {
    const unsigned char* lk = slot;
    const unsigned char* lv = slot + NPART * KBYTES;
    f32x4 sacc[QT][GPS];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt) sacc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < GPS; ++kt) {
      const int row = perm_row<T>(kt, c);
      const int sw = kswz<T>(row, CPR);
      const unsigned char* krow = lk + row * KROWB;
#pragma unroll
      for (int s = 0; s < DSTEPS; ++s) {
        const int off = ((4 * s + g) ^ sw) * 16;
        const uint4 ah = *reinterpret_cast<const uint4*>(krow + off);
#pragma unroll
        for (int t = 0; t < QT; ++t) Mma<T>::run(sacc[t][kt], ah, qreg[t][s]);
        if (SPLIT) {
          const uint4 al = *reinterpret_cast<const uint4*>(krow + KBYTES + off);
#pragma unroll
          for (int t = 0; t < QT; ++t) Mma<T>::run(sacc[t][kt], al, qreg[t][s]);
        }
      }
    }
    const bool ragged = (ch + 1) * KS > r;  // uniform
    uint4 pk[QT];
    float alpha[QT];
    bool need_any = false;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (ragged && ch * KS + perm_row<T>(kt, 4 * g + i) >= r) sacc[t][kt][i] = -INFINITY;
          mx = fmaxf(mx, sacc[t][kt][i]);
        }
      mx = max4g(mx) * scale_log2;
      // lazy rescale: the reference max moves only when the new maximum
      // exceeds it by more than 2^8 (weights stay <= 256, exact in fp32)
      const bool need = mx > m_run[t] + 8.f;
      alpha[t] = need ? fast_exp2(m_run[t] - mx) : 1.f;
      m_run[t] = need ? mx : m_run[t];
      need_any = need_any || need;
      float ls = 0.f;
      f32x4 p[GPS];
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(sacc[t][kt][i], scale_log2, -m_run[t]));
          p[kt][i] = e;
          if (!SPLIT) ls += e;
        }
      if (!SPLIT) l_run[t] = l_run[t] * alpha[t] + ls;
      pk[t] = pack_p<T>(p);
    }
    if (__any(need_any)) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        if (SPLIT) lacc[t] *= alpha[t];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha[t];
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      // lane (g, c) takes V^T row 16*dt + c, ranks g*E .. of the chunk
      const int vr = 16 * dt + c;
      const int voff = vr * VROWB + ((g ^ vswz(vr)) * 16);
      const uint4 a = *reinterpret_cast<const uint4*>(lv + voff);
#pragma unroll
      for (int t = 0; t < QT; ++t) Mma<T>::run(o[t][dt], a, pk[t]);
      if (SPLIT) {
        const uint4 al = *reinterpret_cast<const uint4*>(lv + VBYTES + voff);
#pragma unroll
        for (int t = 0; t < QT; ++t) Mma<T>::run(o[t][dt], al, pk[t]);
      }
    }
    if (SPLIT) {
#pragma unroll
      for (int t = 0; t < QT; ++t) Mma<T>::run(lacc[t], ones, pk[t]);
    }
  };

  // One ring step: chunk i has landed (later ones may stay in flight) and
  // every wave is done with chunk i-1, whose slot takes chunk i+3; then
  // chunk i is used.  Stages run over the passes without a break, so the
  // next pass's first chunks load during this pass's last ones.
  bool active = false;
  auto step = [&](int i, const unsigned char* cur, unsigned char* refill) {
    const int later = nst - 1 - i;  // stages issued after i: min(later, 2)
    if (later >= 2) ring_barrier<2 * PER>();
    else if (later == 1) ring_barrier<PER>();
    else ring_barrier<0>();
    if (i + 3 < nst) issue(i + 3, refill);
    if (active) compute(i % nchunk, cur);
  };
  issue(0, lds0);
  if (nst > 1) issue(1, lds1);
  if (nst > 2) issue(2, lds2);
  for (int pass = 0; pass < passes; ++pass) {
    // this wave's unit of the pass: queries, then fresh softmax state
    const int u = u_begin + pass * kAttWaves + w;
    active = u < u_end;  // wave-uniform
    const int qbase = u * kAttUnit;
    if (active) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int qrow = qbase + 16 * t + c;
        // rows past Lq read row Lq-1 (never stored: each query column is
        // independent), so the loads need no select right after them
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) qreg[t][s] = ld16(q + ((size_t)min(qrow, Lq - 1) * H + h) * D + (4 * s + g) * E);
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
        lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // the ring slot of stage i is i % 4 and a pass has nchunk (a multiple of
    // 4) stages, so every pass starts at slot 0
    const int i0 = pass * nchunk;
    for (int k = 0; k < nchunk; k += kAttRing) {
      step(i0 + k, lds0, lds3);
      step(i0 + k + 1, lds1, lds0);
      step(i0 + k + 2, lds2, lds1);
      step(i0 + k + 3, lds3, lds2);
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int qrow = qbase + 16 * t + c;
        if (qrow < Lq) {
          const float inv = 1.f / (SPLIT ? lacc[t][0] : sum4g(l_run[t]));
          float* dst = o_lin + ((size_t)qrow * H + h) * D + 4 * g;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4*>(dst + 16 * dt) =
                make_float4(o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv, o[t][dt][3] * inv);
        }
      }
    }
  }
}

template <typename T, int D, bool PAGED>
void launch_linear(const Dims& s, const void* q, const void* k_act, const void* v_act, const void* e_k,
                   const void* e_v, void* k_proj, void* v_proj, float* o_lin, int flags, char* ws,
                   const WsLayout& w, const PagedKV<PAGED>& pg, hipStream_t st) {
  // the active tokens the projection contracts: all of them, only the
  // history's (HSA_LIN_HISTORY_PROJ), or only the chunk's, added to the
  // history's given projections into the workspace (HSA_LIN_CHUNK_PROJ)
  const bool chunk = flags & HSA_LIN_CHUNK_PROJ;
  const int t_begin = chunk ? s.Lh : 0;
  const int t_end = (flags & HSA_LIN_HISTORY_PROJ) ? s.Lh : s.L;
  const ProjPlan pp = proj_plan(s, t_end - t_begin);
  float* partial = reinterpret_cast<float*>(ws + w.lin_partial);
  float* kp = chunk ? reinterpret_cast<float*>(ws + w.lin_ksum) : reinterpret_cast<float*>(k_proj);
  float* vp = chunk ? reinterpret_cast<float*>(ws + w.lin_vsum) : reinterpret_cast<float*>(v_proj);
  if (!(flags & HSA_LIN_REUSE_PROJ)) {
    const int n_items = pp.splits * 2 * ((s.H + 1) / 2);
    hipLaunchKernelGGL((lin_project_kernel<T, D, PAGED>), dim3((n_items + 7) / 8 * 8), dim3(kProjThreads), 0, st,
                       reinterpret_cast<const T*>(k_act), reinterpret_cast<const T*>(v_act),
                       reinterpret_cast<const T*>(e_k), reinterpret_cast<const T*>(e_v), s.H, s.L, s.r, pp.splits,
                       t_begin, t_end, partial, pg);
    hipLaunchKernelGGL(lin_reduce_kernel, dim3(2 * s.H, (s.r * D / 4 + 255) / 256), dim3(256), 0, st, partial, s.H, D,
                       s.r, pp.splits, chunk ? reinterpret_cast<const float*>(k_proj) : nullptr,
                       chunk ? reinterpret_cast<const float*>(v_proj) : nullptr, kp, vp);
  }
  if (flags & (HSA_LIN_PROJ_ONLY | HSA_LIN_HISTORY_PROJ)) return;
  // MFMA-ready operands of the attention, then the attention
  T* khi = reinterpret_cast<T*>(ws + w.lin_khi);
  T* klo = reinterpret_cast<T*>(ws + w.lin_klo);
  T* vt = reinterpret_cast<T*>(ws + w.lin_vt);
  T* vlo = reinterpret_cast<T*>(ws + w.lin_vlo);
  hipLaunchKernelGGL((lin_prep_kernel<T>), dim3((pp.rpad * D + 255) / 256, s.H, 2), dim3(256), 0, st, kp, vp, D, s.r,
                     pp.rpad, khi, klo, vt, vlo);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
  const AttendPlan ap = attend_plan(s);
  hipLaunchKernelGGL((lin_attend_kernel<T, D>), dim3(ap.wg_per_head, s.H), dim3(kAttThreads), 0, st,
                     reinterpret_cast<const T*>(q), khi, klo, vt, vlo, s.H, s.Lq, s.r, pp.rpad, ap.units_per_wg,
                     scale_log2, o_lin);
}

}  // namespace
}  // namespace hsa

namespace hsa {
namespace {

template <bool PAGED>
hsa_rc linear_entry(const Dims& s, const void* q, const void* k_act, const void* v_act, const void* e_k,
                    const void* e_v, void* k_proj, void* v_proj, float* o_lin, int32_t flags, void* ws,
                    size_t ws_bytes, hsa_stream stream, const PagedKV<PAGED>& pg) {
  constexpr int kModes = HSA_LIN_REUSE_PROJ | HSA_LIN_PROJ_ONLY | HSA_LIN_HISTORY_PROJ | HSA_LIN_CHUNK_PROJ;
  if (flags & ~kModes) return HSA_ERR_BAD_PARAM;
  if (__builtin_popcount((unsigned)flags) > 1) return HSA_ERR_BAD_PARAM;  // one mode at a time
  // the history / chunk split exists only with the chunk's own keys
  if ((flags & (HSA_LIN_HISTORY_PROJ | HSA_LIN_CHUNK_PROJ)) && !s.split) return HSA_ERR_BAD_PARAM;
  if (!k_proj || !v_proj) return HSA_ERR_NULL_ARG;
  if (!(flags & HSA_LIN_REUSE_PROJ) && ((!PAGED && (!k_act || !v_act)) || !e_k || !e_v)) return HSA_ERR_NULL_ARG;
  if (!(flags & (HSA_LIN_PROJ_ONLY | HSA_LIN_HISTORY_PROJ)) && (!q || !o_lin)) return HSA_ERR_NULL_ARG;
  const WsLayout w = ws_layout(s, 1);
  if (!ws || ws_bytes < w.lin_end) return HSA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  if (s.bf16) {
    if (s.d == 128) launch_linear<bf16_t, 128, PAGED>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, pg, st);
    else launch_linear<bf16_t, 64, PAGED>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, pg, st);
  } else {
    if (s.d == 128) launch_linear<float, 128, PAGED>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, pg, st);
    else launch_linear<float, 64, PAGED>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, wsb, w, pg, st);
  }
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
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
  return linear_entry<false>(s, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, ws, ws_bytes, stream,
                             PagedKV<false>{});
}

extern "C" hsa_rc hsa_linear_branch_paged(const hsa_geom* geom, const void* q, const void* const* page_k,
                                          const void* const* page_v, int32_t n_pages, const int32_t* sel_pages,
                                          const void* e_k, const void* e_v, void* k_proj, void* v_proj,
                                          float* o_lin, int32_t flags, void* ws, size_t ws_bytes,
                                          hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  // a contraction step (at most 32 tokens) must span at most two pages
  if (s.Lp < 32) return HSA_ERR_BAD_SHAPE;
  PagedKV<true> pg;
  for (int j = 0; j < kMaxPages; ++j) pg.pk.p[j] = pg.pv.p[j] = nullptr;
  if (!(flags & HSA_LIN_REUSE_PROJ)) {
    if (!page_k || !page_v || !sel_pages) return HSA_ERR_NULL_ARG;
    if (n_pages < 1 || n_pages > HSA_MAX_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
    for (int j = 0; j < n_pages; ++j) {
      if (!page_k[j] || !page_v[j]) return HSA_ERR_NULL_ARG;
      pg.pk.p[j] = page_k[j];
      pg.pv.p[j] = page_v[j];
    }
  }
  pg.sel = sel_pages;
  pg.n_pages = n_pages;
  pg.Lp = s.Lp;
  return linear_entry<true>(s, q, nullptr, nullptr, e_k, e_v, k_proj, v_proj, o_lin, flags, ws, ws_bytes, stream,
                            pg);
}

extern "C" hsa_rc hsa_linear_branch_paged_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                                 const void* const* page_v_table, int32_t n_pages,
                                                 const int32_t* sel_pages, const void* e_k, const void* e_v,
                                                 void* k_proj, void* v_proj, float* o_lin, int32_t flags, void* ws,
                                                 size_t ws_bytes, hsa_stream stream) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (s.Lp < 32) return HSA_ERR_BAD_SHAPE;
  PagedKV<true> pg;
  for (int j = 0; j < kMaxPages; ++j) pg.pk.p[j] = pg.pv.p[j] = nullptr;
  if (!(flags & HSA_LIN_REUSE_PROJ)) {
    if (!page_k_table || !page_v_table || !sel_pages) return HSA_ERR_NULL_ARG;
    if (n_pages < 1 || n_pages > HSA_MAX_BANK_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
    pg.dk = page_k_table;
    pg.dv = page_v_table;
  }
  pg.sel = sel_pages;
  pg.n_pages = n_pages;
  pg.Lp = s.Lp;
  return linear_entry<true>(s, q, nullptr, nullptr, e_k, e_v, k_proj, v_proj, o_lin, flags, ws, ws_bytes, stream,
                            pg);
}
