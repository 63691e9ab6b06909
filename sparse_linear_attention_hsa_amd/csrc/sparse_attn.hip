// S5 -- block-sparse attention.  WorldAttention paper, section 3.3 "Sparse
// branch" and appendix A.1.3: attention at token resolution, restricted to
// the (query block, key block) pairs that were selected; for query block i of
// head h, O = softmax(Q_i K_S^T / sqrt(d)) V_S over exactly the tokens S of
// its selected key blocks.
//
// Design (gfx950, wave64, 16x16 matrix cores):
//  * Work is cut in 16-token key granules.  A row (head, query block) owns
//    count*B/16 granules; rows longer than a segment are split into balanced
//    segments so that every workgroup gets a similar amount of work even when
//    heads keep very different numbers of blocks.  A tiny plan kernel lays the
//    segments out; segments of a split row write un-normalised partial
//    outputs with their running max and sum, merged exactly by a combine
//    kernel (fixed order, no atomics).
//  * Workgroup = NW waves; wave w owns QPW (at most two) 16-row query tiles
//    of the block, which keeps a wave at 168 registers: three waves per SIMD.
//    Per step it stages KS keys (32 for bf16, 16 for f32) of K (row-major)
//    and of V (d-major, as the gather lays V out) in LDS, in a ring of two
//    or three stages fed by direct global->LDS loads,
//    and every wave computes S^T = K Q^T (keys on the rows, so each lane owns
//    one query column), an online softmax per query, and O^T += V^T P^T.
//    Keeping queries on the lane-column axis puts the softmax state and the
//    output column of a query in the same lane: no cross-lane rescaling.
//  * XCD-aware item order: items are laid out head by head and, inside a
//    head, by the key range they cover; each XCD runs one contiguous range of
//    them, so the workgroups running together on an XCD read the same key and
//    value blocks and share them through that XCD's L2.  Heads run in phases
//    (all XCDs on a few heads at a time), so that what the L2 misses fetch
//    stays within the last-level cache.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kPlanThreads = 1024;

// Inclusive prefix sum over the 1024 threads of the workgroup: a shuffle
// scan inside each wave, then the 16 wave totals (buf holds >= 16 ints).
__device__ int scan_incl_1024(int v, int* buf) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == kWave - 1) buf[wave] = v;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < wave; ++k) before += buf[k];
  __syncthreads();  // buf may be reused by the caller
  return v + before;
}

// Work items are (row, segment) pairs; a row (head h, query block i) with G
// granules gets nseg = ceil(G / seg_granules) balanced segments.  Items are
// laid out head by head and, inside a head, by the key range they cover: the
// key block at the middle of the segment, in buckets of 2^bucket_shift
// blocks.  Each XCD runs one contiguous range of items, so the workgroups
// that run together on it read the same key and value blocks, and those stay
// in its L2.  (Ordered by segment index instead, a head's workgroups spread
// over its whole key range; in a simulation of the C1 dispatch the L2 hit
// rate was 30% against 49% ordered by key range.)  Inside a bucket the order
// is whatever the LDS atomics give: no result depends on it, since every
// item writes its own output rows or its own partial slot.
// items[k] = {row, first granule, granules, partial slot or -1};
// rowinfo[row] = {segments, first slot}; meta = {items, slots}.
constexpr int kMaxPlanRows = HSA_MAX_ROWS;
constexpr int kMaxPlanSegs = kPlanMaxSegs;
constexpr int kMaxPlanKeys = kPlanMaxBuckets;  // (head, key bucket) pairs
static_assert(kMaxPlanKeys <= 2 * kPlanThreads, "the bucket scan takes two entries per thread");
constexpr int kPlanBatch = 4;       // items per thread whose block-id loads are in flight together

__global__ __launch_bounds__(kPlanThreads) void sparse_plan_kernel(
    const int32_t* __restrict__ blk_count, const int32_t* __restrict__ blk_idx, int rows, int nQB, int nKB, int gpb,
    int gps, int seg_granules, int bucket_shift, int heads_per_phase, int4* __restrict__ items,
    int2* __restrict__ rowinfo, int* __restrict__ meta) {
  __shared__ short nseg_s[kMaxPlanRows];
  __shared__ int per_s[kMaxPlanRows];
  __shared__ int gran_s[kMaxPlanRows];   // granules of every row
  __shared__ int slot_s[kMaxPlanRows];
  __shared__ int first_s[kMaxPlanRows];  // the row's first item in row order
  __shared__ int off_s[kMaxPlanKeys];    // items per bucket, then each bucket's next place
  __shared__ int buf[kPlanThreads];
  __shared__ int carry_slot, carry_item;
  const int t = threadIdx.x;
  const int nb = ((nKB - 1) >> bucket_shift) + 1;  // buckets per head
  const int nkeys = (rows / nQB) * nb;
  for (int k = t; k < nkeys; k += kPlanThreads) off_s[k] = 0;
  if (t == 0) carry_slot = carry_item = 0;
  __syncthreads();
  // 1) segments of every row; partial slots are contiguous per split row
  for (int base = 0; base < rows; base += kPlanThreads) {
    const int row = base + t;
    int nseg = 0, per = 0, G_row = 0;
    if (row < rows) {
      int n = blk_count[row];
      n = n < 0 ? 0 : (n > nKB ? nKB : n);
      const int G = n * gpb;
      G_row = G;
      if (G > 0) {
        nseg = (G + seg_granules - 1) / seg_granules;
        per = (G + nseg - 1) / nseg;
        per = (per + gps - 1) / gps * gps;
        nseg = (G + per - 1) / per;
      }
    }
    const int nslot = nseg > 1 ? nseg : 0;
    const int cs = scan_incl_1024(nslot, buf) - nslot;
    const int ci = scan_incl_1024(nseg, buf) - nseg;
    if (row < rows) {
      nseg_s[row] = (short)nseg;
      per_s[row] = per;
      gran_s[row] = G_row;
      slot_s[row] = carry_slot + cs;
      first_s[row] = carry_item + ci;
      rowinfo[row] = make_int2(nseg, carry_slot + cs);
    }
    __syncthreads();
    if (t == kPlanThreads - 1) {
      carry_slot += cs + nslot;
      carry_item += ci + nseg;
    }
    __syncthreads();
  }
  const int n_items = carry_item;
  if (t == 0) {
    meta[0] = n_items;
    meta[1] = carry_slot;
  }
  // item k (in row order) -> its row: the last row whose first item is <= k
  // (rows without items share the next row's first item, so the last such
  // row is the one that has items)
  auto row_of = [&](int k) {
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first_s[mid] <= k) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  // the (head, key bucket) of items k0 + j * kPlanThreads, with all their
  // block-id loads issued before the first is used
  auto keys_of = [&](int k0, int* key, int* row, int* sg) {
    int b[kPlanBatch];
#pragma unroll
    for (int j = 0; j < kPlanBatch; ++j) {
      const int k = k0 + j * kPlanThreads;
      b[j] = 0;
      row[j] = 0;
      sg[j] = 0;
      if (k < n_items) {
        row[j] = row_of(k);
        sg[j] = k - first_s[row[j]];
        const int per = per_s[row[j]];
        const int g0 = sg[j] * per;
        const int cnt = min(per, gran_s[row[j]] - g0);
        b[j] = blk_idx[(size_t)row[j] * nKB + (g0 + cnt / 2) / gpb];
      }
    }
#pragma unroll
    for (int j = 0; j < kPlanBatch; ++j) {
      const int bj = b[j] < 0 ? 0 : (b[j] >= nKB ? nKB - 1 : b[j]);  // any id orders somewhere
      key[j] = (row[j] / nQB) * nb + (bj >> bucket_shift);
    }
  };
  // 2) items per bucket
  for (int k0 = t; k0 < n_items; k0 += kPlanBatch * kPlanThreads) {
    int key[kPlanBatch], row[kPlanBatch], sg[kPlanBatch];
    keys_of(k0, key, row, sg);
#pragma unroll
    for (int j = 0; j < kPlanBatch; ++j)
      if (k0 + j * kPlanThreads < n_items) atomicAdd(&off_s[key[j]], 1);
  }
  __syncthreads();
  // 3) exclusive scan of the counts in (head, bucket) order (two entries per thread)
  {
    const int a0 = 2 * t < nkeys ? off_s[2 * t] : 0;
    const int a1 = 2 * t + 1 < nkeys ? off_s[2 * t + 1] : 0;
    const int incl = scan_incl_1024(a0 + a1, buf);
    if (2 * t < nkeys) off_s[2 * t] = incl - a0 - a1;
    if (2 * t + 1 < nkeys) off_s[2 * t + 1] = incl - a1;
  }
  __syncthreads();
  // the first item of every head (and the item count after the last head),
  // and how many per-XCD indices the phases use (a workgroup past them has
  // no item, whatever its phase)
  const int nheads = rows / nQB;
  if (t <= nheads) meta[2 + t] = t < nheads ? off_s[t * nb] : n_items;
  if (t == 0) {
    int k_used = 0;
    for (int h0 = 0; h0 < nheads; h0 += heads_per_phase) {
      const int hb = min(h0 + heads_per_phase, nheads);
      k_used += ceil_div((hb < nheads ? off_s[hb * nb] : n_items) - off_s[h0 * nb], 8);
    }
    meta[kPlanMetaInts - 1] = k_used;
  }
  __syncthreads();  // the head starts are read before step 4 advances off_s
  // 4) every item to the next place of its bucket
  for (int k0 = t; k0 < n_items; k0 += kPlanBatch * kPlanThreads) {
    int key[kPlanBatch], row[kPlanBatch], sg[kPlanBatch];
    keys_of(k0, key, row, sg);
#pragma unroll
    for (int j = 0; j < kPlanBatch; ++j) {
      if (k0 + j * kPlanThreads < n_items) {
        const int r = row[j], per = per_s[r], nseg = nseg_s[r];
        const int pos = atomicAdd(&off_s[key[j]], 1);
        items[pos] = make_int4(r, sg[j] * per, min(per, gran_s[r] - sg[j] * per), nseg > 1 ? slot_s[r] + sg[j] : -1);
      }
    }
  }
}

// Partial outputs of split rows: each segment's output normalised by its own
// softmax sum, so every element is a convex combination of values (|o| <=
// max |v|).  bf16 workloads keep them in half precision (2^-11 relative,
// against the 2^-9 of the bf16 operands), halving the bytes the segments
// write and the merge reads; float32 workloads keep float32.
template <typename T> struct PartOf { using type = float; };
template <> struct PartOf<bf16_t> { using type = _Float16; };
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store4(float* p, const f32x4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(_Float16* p, const f32x4& v) {
  *reinterpret_cast<half4_t*>(p) = __builtin_convertvector(v, half4_t);
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const _Float16* p) {
  const half4_t h = *reinterpret_cast<const half4_t*>(p);
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}

// Work item of workgroup bid.  Heads run in phases of heads_per_phase: the
// XCDs (which receive consecutive workgroup ids round-robin) all take items
// of one phase, each XCD one contiguous range of them, before the next
// phase's items.  meta[2 + h] is the first item of head h (meta[2 + H] the
// item count); -1 for a surplus workgroup.
__device__ __forceinline__ int phased_remap(int bid, const int* meta, int H, int heads_per_phase) {
  const int x = bid & 7, k = bid >> 3;
  if (k >= meta[kPlanMetaInts - 1]) return -1;  // past every phase: one load, no walk
  int k0 = 0;  // first per-XCD index of the phase
  for (int h0 = 0; h0 < H; h0 += heads_per_phase) {
    const int a = meta[2 + h0], b = meta[2 + min(h0 + heads_per_phase, H)];
    const int per = ceil_div(b - a, 8);
    if (k < k0 + per) {
      const int item = a + x * per + (k - k0);
      return item < b ? item : -1;
    }
    k0 += per;
  }
  return -1;
}

// LDS staging of one step (KS keys), written by direct global->LDS loads
// (each wave instruction writes 1 KB: 64 lanes x 16 bytes, contiguous).
//  * K: rows of D elements, 16-byte chunks swizzled by kswz (common.h).
//  * V: the step's granules as regions [granule][part][D rows][16 bytes];
//    region g is exactly what lane group g reads for the V^T operand.

// FULL: every wave owns exactly QPW query tiles (B == 16*NW*QPW), so the tile
// loops carry no run-time guards and the matrix-core chains stay branch-free.
template <typename T, int D, int NW, int QPW, int WPE, int RING, bool FULL, bool PAGED>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void sparse_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k_act, const T* __restrict__ v_act,
    const int32_t* __restrict__ blk_idx, const int4* __restrict__ items, const int* __restrict__ meta,
    int H, int B, int Bk, int L, int nKB, int nQB, int heads_per_phase, float scale_log2,
    float* __restrict__ o_sp, typename PartOf<T>::type* __restrict__ part_o, float* __restrict__ part_ml,
    PagedKV<PAGED> pg) {
  constexpr int E = Vec<T>::N;          // elements per 16-byte chunk
  constexpr int KS = Mma<T>::K;         // keys per step
  constexpr int GPS = KS / 16;          // granules per step
  constexpr int CPR = D / E;            // chunks per key row
  constexpr int DSTEPS = D / KS;        // contraction steps over d in S^T = K Q^T
  constexpr int DT = D / 16;            // output d-tiles
  constexpr int PV = 16 / E;            // 16-byte parts per granule row of V
  constexpr int KBYTES = KS * CPR * 16; // K stage bytes
  constexpr int VBYTES = GPS * PV * D * 16;
  constexpr int KINST = KBYTES / 1024;  // 1 KB direct-load instructions
  constexpr int VINST = VBYTES / 1024;
  constexpr int ROWS_PER_INST = 64 / CPR;
  constexpr float kLazy = 8.f;          // rescale only when the row max grows by more than 2^8 (log2 units)
  static_assert(RING == 2 || RING == 3, "staging ring depth");

  // RING stages of K and V, each buffer its own object so the compiler can
  // tell an operand read of one stage from the loads still in flight into
  // the others (a third buffer goes unused when RING == 2)
  __shared__ __align__(1024) unsigned char lds_k0[KBYTES], lds_k1[KBYTES], lds_k2[RING == 3 ? KBYTES : 16];
  __shared__ __align__(1024) unsigned char lds_v0[VBYTES], lds_v1[VBYTES], lds_v2[RING == 3 ? VBYTES : 16];

  const int item = phased_remap(blockIdx.x, meta, H, heads_per_phase);
  if (item < 0) return;
  const int4 it = items[item];
  const int row = it.x, g0 = it.y, gcount = it.z, slot = it.w;
  const int h = row / nQB, qb = row % nQB;
  const int gpb = Bk / 16;  // granules per key block (query tiles are B rows)

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave index, kept in a scalar register
  const int g = lane >> 4, c = lane & 15;
  const int QT = B / 16;
  const int ntile = FULL ? QPW : min(QPW, QT - w * QPW);  // wave-uniform

  // The segment's block ids, one per lane (the plan keeps a segment within
  // 64 blocks).
  const int b0 = g0 / gpb;
  const int nblk = gcount > 0 ? (g0 + gcount - 1) / gpb - b0 + 1 : 0;
  const int blk_lane = lane < nblk ? blk_idx[(size_t)row * nKB + b0 + lane] : -1;
  // paged: each lane's block as its block within its page (-1 for an invalid
  // id) and that page's K and V base pointers, held in registers so that a
  // granule's page costs register reads, not a memory wait; an invalid id
  // takes the first selected page
  int lblk_lane = -1;
  uint32_t kp_lo = 0, kp_hi = 0, vp_lo = 0, vp_hi = 0;
  if constexpr (PAGED) {
    const int bpp = pg.Lp / Bk;
    const bool valid = blk_lane >= 0 && blk_lane < nKB;
    const int ps = valid ? blk_lane / bpp : 0;
    lblk_lane = valid ? blk_lane - ps * bpp : -1;
    int page = pg.sel[ps];
    page = page < 0 ? 0 : (page >= pg.n_pages ? pg.n_pages - 1 : page);
    const uint64_t kp = reinterpret_cast<uint64_t>(pg.kpage(page));
    const uint64_t vp = reinterpret_cast<uint64_t>(pg.vpage(page));
    kp_lo = (uint32_t)kp;
    kp_hi = (uint32_t)(kp >> 32);
    vp_lo = (uint32_t)vp;
    vp_hi = (uint32_t)(vp >> 32);
  }
  auto ptr_of = [](uint32_t lo, uint32_t hi) {
    return reinterpret_cast<const T*>((uint64_t)lo | ((uint64_t)hi << 32));
  };

  // Q^T operand: lane (g, c) holds Q[row c of tile][chunk 4s+g] for step s.
  uint4 qreg[QPW][DSTEPS];
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    if (t < ntile) {
      const size_t qrow = (size_t)qb * B + (w * QPW + t) * 16 + c;
      const T* qp = q + (qrow * H + h) * D;
#pragma unroll
      for (int s = 0; s < DSTEPS; ++s) qreg[t][s] = ld16(qp + (4 * s + g) * E);
    }
  }

  // Output accumulators, plus one more 16-row tile per query tile fed by an
  // all-ones operand: its rows are the running softmax denominators (the sum
  // of exactly the bf16-rounded weights the numerator uses), in every lane
  // group, with no cross-lane reduction.  The running max starts at a finite
  // -1e30, so weights of masked keys are exp2(-inf) = 0 without a special case.
  f32x4 o[QPW][DT], lacc[QPW];
  float m_run[QPW], thr[QPW];
  const float inv_scale = 1.f / scale_log2;
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    m_run[t] = -1e30f;
    thr[t] = (-1e30f + kLazy) * inv_scale;
    lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = sizeof(T) == 2 ? make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u)
                                    : make_uint4(0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u);

  const int nsub = (gcount + GPS - 1) / GPS;
  const T* kh = k_act + (size_t)h * L * D;
  const T* vh = v_act + (size_t)h * (L / 16) * D * 16;
  // Direct loads go through buffer resources over the head's K and V: a lane's
  // address is one 32-bit byte offset and the granule's part a scalar offset
  // (a global address takes a 64-bit register pair per load).  A head's
  // active K/V is at most HSA_MAX_KBLOCKS * 192 * 128 * 4 bytes, well within
  // 32 bits.
  const int head_bytes = (int)((size_t)L * D * sizeof(T));
  // paged: one head of one page, K [Lp][d] or V [Lp/16][d][16]
  const int page_head_bytes = PAGED ? (int)((size_t)pg.Lp * D * sizeof(T)) : 0;
  const size_t page_head_elems = PAGED ? (size_t)h * pg.Lp * D : 0;

  // per-lane parts of the direct-load addresses (element offsets from the
  // start of the granule); only the granule's key offset changes per step
  constexpr int KPW = (KINST + NW - 1) / NW, VPW = (VINST + NW - 1) / NW;
  // direct loads every wave issues per stage, at least
  constexpr int PER_STAGE = KINST / NW + VINST / NW;
  int koff[KPW], kgran[KPW], voff[VPW], vgran[VPW];
#pragma unroll
  for (int ii = 0; ii < KPW; ++ii) {
    const int i = ii * NW + w;
    const int rho = i * ROWS_PER_INST + lane / CPR;
    const int chunk = (lane % CPR) ^ kswz<T>(rho, CPR);
    kgran[ii] = rho / 16;
    koff[ii] = (rho % 16) * D + chunk * E;
  }
#pragma unroll
  for (int ii = 0; ii < VPW; ++ii) {
    const int i = ii * NW + w;
    const int region = i / (D / 64);
    const int rowv = (i % (D / 64)) * 64 + lane;
    vgran[ii] = region / PV;
    voff[ii] = rowv * 16 + (region % PV) * E;
  }

  // Issue cursor over the segment's granules (scalar state): stages are
  // issued strictly in order, GPS granules each.
  int cur_blk = 0, cur_gran = g0 - b0 * gpb, issued = 0;
  // Stage the next GPS granules into (lk, lv); returns their validity bits.
  auto issue = [&](unsigned char* lk, unsigned char* lv) -> unsigned {
    int kofs[GPS];
    uint32_t kb_lo[GPS], kb_hi[GPS], vb_lo[GPS], vb_hi[GPS];  // paged: the granule's page
    unsigned mask = 0;
#pragma unroll
    for (int j = 0; j < GPS; ++j) {
      int key = -1;
      const int src = issued < gcount ? cur_blk : 0;  // lane of the granule's block
      if (issued < gcount) {
        if constexpr (PAGED) {
          const int lb = __builtin_amdgcn_readlane(lblk_lane, cur_blk);
          if (lb >= 0) key = lb * Bk + cur_gran * 16;
        } else {
          const int blk = __builtin_amdgcn_readlane(blk_lane, cur_blk);
          if (blk >= 0 && blk < nKB) key = blk * Bk + cur_gran * 16;
        }
      }
      if constexpr (PAGED) {
        kb_lo[j] = __builtin_amdgcn_readlane(kp_lo, src);
        kb_hi[j] = __builtin_amdgcn_readlane(kp_hi, src);
        vb_lo[j] = __builtin_amdgcn_readlane(vp_lo, src);
        vb_hi[j] = __builtin_amdgcn_readlane(vp_hi, src);
      }
      // a masked granule (past the segment or an invalid block id) loads the
      // head's first granule (paged: of its page or the first selected one):
      // its scores are set to -inf, so it adds nothing
      kofs[j] = key >= 0 ? key : 0;
      mask |= (key >= 0 ? 1u : 0u) << j;
      ++issued;
      if (++cur_gran == gpb) {
        cur_gran = 0;
        ++cur_blk;
      }
    }
#pragma unroll
    for (int ii = 0; ii < KPW; ++ii) {
      const int i = ii * NW + w;
      if (KINST % NW != 0 && i >= KINST) break;
      const int kg = kofs[kgran[ii]];
      if constexpr (PAGED) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane(kb_lo[kgran[ii]]);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(kb_hi[kgran[ii]]);
        // a page a device table holds no buffer for: an empty range, so the loads return zeros
        buffer_load_lds16(ptr_of(lo, hi) + page_head_elems, (lo | hi) ? page_head_bytes : 0, lk + i * 1024,
                          koff[ii] * (int)sizeof(T), kg * D * (int)sizeof(T));
      } else {
        buffer_load_lds16(kh, head_bytes, lk + i * 1024, koff[ii] * (int)sizeof(T), kg * D * (int)sizeof(T));
      }
    }
#pragma unroll
    for (int ii = 0; ii < VPW; ++ii) {
      const int i = ii * NW + w;
      if (VINST % NW != 0 && i >= VINST) break;
      const int kg = kofs[vgran[ii]];
      if constexpr (PAGED) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane(vb_lo[vgran[ii]]);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(vb_hi[vgran[ii]]);
        buffer_load_lds16(ptr_of(lo, hi) + page_head_elems, (lo | hi) ? page_head_bytes : 0, lv + i * 1024,
                          voff[ii] * (int)sizeof(T), kg * D * (int)sizeof(T));
      } else {
        buffer_load_lds16(vh, head_bytes, lv + i * 1024, voff[ii] * (int)sizeof(T), kg * D * (int)sizeof(T));
      }
    }
    return mask;
  };

  constexpr unsigned kAllValid = (1u << GPS) - 1;
  // S^T products of one granule half kt (both query tiles share each K read)
  auto products = [&](const unsigned char* lk, f32x4 (&sacc)[QPW][GPS], int kt) {
    const int rho = perm_row<T>(kt, c);
    const unsigned char* krow = lk + rho * CPR * 16;
    const int sw = kswz<T>(rho, CPR);
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(krow + (((4 * s + g) ^ sw) * 16));
#pragma unroll
      for (int t = 0; t < QPW; ++t)
        if (FULL || t < ntile) Mma<T>::run(sacc[t][kt], a, qreg[t][s]);
    }
  };
  // weight of one score under the reference max of tile t
  auto wt = [&](float sc, int t) { return fast_exp2(fmaf(sc, scale_log2, -m_run[t])); };
  // packed weights of granule half kt: bf16 pairs for bf16, raw floats for f32
  auto weights_half = [&](const f32x4& sh, int t) -> uint2 {
    return make_uint2(pack2_bf16(wt(sh[0], t), wt(sh[1], t)), pack2_bf16(wt(sh[2], t), wt(sh[3], t)));
  };
  auto compute = [&](const unsigned char* lk, const unsigned char* lv, unsigned mask) {
    if (!(FULL || w * QPW < QT)) return;
    f32x4 sacc[QPW][GPS];
#pragma unroll
    for (int t = 0; t < QPW; ++t)
#pragma unroll
      for (int kt = 0; kt < GPS; ++kt) sacc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // bf16: the first half's products, then its weights under the current
    // reference max while the second half's products run on the matrix
    // cores; the (rare) move of the reference max below recomputes them.
    uint2 ph[QPW];
    products(lk, sacc, 0);
    if constexpr (GPS == 2) {
#pragma unroll
      for (int t = 0; t < QPW; ++t)
        if (FULL || t < ntile) ph[t] = weights_half(sacc[t][0], t);
      products(lk, sacc, 1);
    }
    if (mask != kAllValid) {
      // masked keys, only on a ragged or invalid step (wave-uniform test):
      // lane group g holds keys of granule g/2 (bf16) or granule 0 (f32);
      // their scores become -inf and the first half's weights exactly 0
      const bool ok = (mask >> (GPS == 2 ? (g >> 1) : 0)) & 1u;
#pragma unroll
      for (int t = 0; t < QPW; ++t) {
#pragma unroll
        for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[t][kt][i] = ok ? sacc[t][kt][i] : -INFINITY;
        if constexpr (GPS == 2) ph[t] = ok ? ph[t] : make_uint2(0u, 0u);
      }
    }
    // Lazy test, lane-local: a query's weights can exceed 2^kLazy only if one
    // of this lane's raw scores exceeds thr = (m + kLazy) / scale.  Only then
    // is the max reduced across the four lane groups (uniform per query).
    bool up = false;
#pragma unroll
    for (int t = 0; t < QPW; ++t)
      if (FULL || t < ntile) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[t][kt][i]);
        up = up || mx > thr[t];
      }
    if (__any(up)) {  // rare: the reference max moves
#pragma unroll
      for (int t = 0; t < QPW; ++t)
        if (FULL || t < ntile) {
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < GPS; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[t][kt][i]);
          mx = max4g(mx) * scale_log2;
          if (mx > m_run[t] + kLazy) {  // uniform across the lane groups of a query
            const float alpha = fast_exp2(m_run[t] - mx);
            lacc[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
            m_run[t] = mx;
            thr[t] = (mx + kLazy) * inv_scale;
            if constexpr (GPS == 2) ph[t] = weights_half(sacc[t][0], t);
          }
        }
    }
    uint4 pk[QPW];
#pragma unroll
    for (int t = 0; t < QPW; ++t)
      if (FULL || t < ntile) {
        if constexpr (GPS == 2) {
          const uint2 p1 = weights_half(sacc[t][1], t);
          pk[t] = make_uint4(ph[t].x, ph[t].y, p1.x, p1.y);
        } else {
          pk[t] = make_uint4(__float_as_uint(wt(sacc[t][0][0], t)), __float_as_uint(wt(sacc[t][0][1], t)),
                             __float_as_uint(wt(sacc[t][0][2], t)), __float_as_uint(wt(sacc[t][0][3], t)));
        }
      }
    const unsigned char* vreg = lv + g * (D * 16);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 a = *reinterpret_cast<const uint4*>(vreg + (16 * dt + c) * 16);
#pragma unroll
      for (int t = 0; t < QPW; ++t)
        if (FULL || t < ntile) Mma<T>::run(o[t][dt], a, pk[t]);
    }
#pragma unroll
    for (int t = 0; t < QPW; ++t)
      if (FULL || t < ntile) Mma<T>::run(lacc[t], ones, pk[t]);
  };

  // One step: wait for this stage (this wave's loads, then every wave's),
  // refill the ring slot that the previous step finished with, compute.
  auto step = [&](int sub, const unsigned char* lk, const unsigned char* lv, unsigned mask,
                  unsigned char* nk, unsigned char* nv, unsigned& nmask) {
    if (RING == 3 && sub + 1 < nsub) ring_barrier<PER_STAGE>();  // the next stage may stay in flight
    else ring_barrier<0>();
    if (sub + RING - 1 < nsub) nmask = issue(nk, nv);
    compute(lk, lv, mask);
  };

  unsigned m0 = 0, m1 = 0, m2 = 0;
  if (nsub > 0) m0 = issue(lds_k0, lds_v0);
  if (RING == 3) {
    if (nsub > 1) m1 = issue(lds_k1, lds_v1);
    for (int sub = 0; sub < nsub; sub += 3) {
      step(sub, lds_k0, lds_v0, m0, lds_k2, lds_v2, m2);
      if (sub + 1 < nsub) step(sub + 1, lds_k1, lds_v1, m1, lds_k0, lds_v0, m0);
      if (sub + 2 < nsub) step(sub + 2, lds_k2, lds_v2, m2, lds_k1, lds_v1, m1);
    }
  } else {
    for (int sub = 0; sub < nsub; sub += 2) {
      step(sub, lds_k0, lds_v0, m0, lds_k1, lds_v1, m1);
      if (sub + 1 < nsub) step(sub + 1, lds_k1, lds_v1, m1, lds_k0, lds_v0, m0);
    }
  }

  // epilogue
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    if (t < ntile) {
      const float l_tot = lacc[t][0];  // every row of the ones tile holds the denominator
      const int r = (w * QPW + t) * 16 + c;  // query row inside the block
      if (slot < 0) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* dst = o_sp + (((size_t)qb * B + r) * H + h) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 v = o[t][dt] * inv;
          *reinterpret_cast<float4*>(dst + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        auto* dst = part_o + ((size_t)slot * B + r) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4(dst + 16 * dt, o[t][dt] * inv);
        if (g == 0) {
          part_ml[((size_t)slot * B + r) * 2 + 0] = m_run[t];
          part_ml[((size_t)slot * B + r) * 2 + 1] = l_tot;
        }
      }
    }
  }
}

// Merge the partial outputs of split rows (fixed segment order); rows with
// no selected block get zeros.  kCombParts workgroups share a row, each with
// a quarter of its query rows and all their columns, so a wave reads whole
// 128-byte lines of the half-precision partials.  (Split by columns instead,
// each workgroup read half of every line, and the four workgroups of a row
// run on different XCDs, so each line came from memory twice.)  The
// per-segment weights l_s exp2(m_s - M) / sum_s' l_s' exp2(m_s' - M) (for
// outputs normalised per segment) go through LDS, then every thread streams
// its four-column groups once.
constexpr int kCombThreads = 256;
constexpr int kCombParts = 4;

template <int D, typename PartT>
__global__ __launch_bounds__(kCombThreads) void sparse_combine_kernel(
    const int2* __restrict__ rowinfo, const PartT* __restrict__ part_o, const float* __restrict__ part_ml,
    int H, int B, int nQB, float* __restrict__ o_sp) {
  // (running max, sum) of every segment row, then (weight, -) in place;
  // max_segs x B entries (dynamic)
  extern __shared__ float2 ml[];
  const int row = blockIdx.x / kCombParts, part = blockIdx.x % kCombParts;
  const int2 ri = rowinfo[row];
  const int nseg = ri.x, s0 = ri.y;
  if (nseg == 1) return;
  const int h = row / nQB, qb = row % nQB;
  if (nseg > 1) {
    // all (max, sum) pairs of the row in one parallel step
    const float2* pml = reinterpret_cast<const float2*>(part_ml) + (size_t)s0 * B;
    for (int e = threadIdx.x; e < nseg * B; e += kCombThreads) ml[e] = pml[e];
    __syncthreads();
    for (int r = threadIdx.x; r < B; r += kCombThreads) {
      float M = -INFINITY;
      for (int sg = 0; sg < nseg; ++sg) M = fmaxf(M, ml[sg * B + r].x);
      if (M == -INFINITY) M = 0.f;  // (running maxima start at -1e30; kept for any caller)
      float den = 0.f;
      for (int sg = 0; sg < nseg; ++sg) {
        const float2 v = ml[sg * B + r];
        const float wv = exp2f(v.x - M) * v.y;
        ml[sg * B + r].x = wv;
        den += wv;
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      for (int sg = 0; sg < nseg; ++sg) ml[sg * B + r].x *= inv;
    }
  }
  __syncthreads();
  // Three float4 columns per thread and pass, with the loads of up to four
  // segments of all three in flight together; each column still sums its
  // segments in segment order.
  constexpr int U = 3;
  constexpr int CW = D / 4;  // four-column groups per query row
  const int prow = B / kCombParts;  // query rows of this workgroup
  const int total = prow * CW;
  const size_t seg_stride = (size_t)B * D;  // elements between the partials of consecutive segments
  const PartT* base = part_o + (size_t)s0 * B * D + (size_t)part * prow * D;
  for (int e0 = threadIdx.x; e0 < total; e0 += U * kCombThreads) {
    int rr[U];
    bool ok[U];
    const PartT* src[U];
    float4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kCombThreads;
      ok[u] = e < total;
      const int ec = ok[u] ? e : 0;  // clamped: a column past the end reads column 0 and is not stored
      rr[u] = part * prow + ec / CW;
      src[u] = base + (size_t)(ec / CW) * D + 4 * (ec % CW);
      acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    int sg = 0;
    for (; sg + 4 <= nseg; sg += 4) {
      float4 v[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[u][k] = load4(src[u] + (size_t)(sg + k) * seg_stride);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float wv = ml[(sg + k) * B + rr[u]].x;
          acc[u].x += wv * v[u][k].x; acc[u].y += wv * v[u][k].y;
          acc[u].z += wv * v[u][k].z; acc[u].w += wv * v[u][k].w;
        }
    }
    for (; sg < nseg; ++sg) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = load4(src[u] + (size_t)sg * seg_stride);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wv = ml[sg * B + rr[u]].x;
        acc[u].x += wv * v[u].x; acc[u].y += wv * v[u].y; acc[u].z += wv * v[u].z; acc[u].w += wv * v[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) {
        const int e = e0 + u * kCombThreads;
        reinterpret_cast<float4*>(o_sp + (((size_t)qb * B + rr[u]) * H + h) * D)[e % CW] = acc[u];
      }
    }
  }
}

template <typename T, int D, int NW, int QPW, bool PAGED>
void launch_attn(const Dims& s, const SparsePlan& pl, const void* q, const void* k_act, const void* v_act,
                 const int32_t* idx, const int4* items, const int* meta, float* o_sp,
                 void* po, float* pml, const PagedKV<PAGED>& pg, hipStream_t st) {
  using PartT = typename PartOf<T>::type;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)s.d);
  // bf16: two query tiles per wave fit 168 registers, three waves per SIMD
  constexpr int WPE = sizeof(T) == 2 ? (QPW <= 2 ? 3 : 2) : 1;
  // a third stage only where it still leaves room for four workgroups per CU
  constexpr int STAGE = 2 * Mma<T>::K * D * (int)sizeof(T);
  constexpr int RING = 3 * STAGE <= 24576 ? 3 : 2;
  if (s.B == 16 * NW * QPW)
    hipLaunchKernelGGL((sparse_attn_kernel<T, D, NW, QPW, WPE, RING, true, PAGED>), dim3(pl.grid), dim3(NW * kWave),
                       0, st, reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k_act),
                       reinterpret_cast<const T*>(v_act), idx, items, meta, s.H, s.B, s.Bk, s.L, s.nKB, s.nQB, pl.heads_per_phase,
                       scale_log2, o_sp, static_cast<PartT*>(po), pml, pg);
  else
  hipLaunchKernelGGL((sparse_attn_kernel<T, D, NW, QPW, WPE, RING, false, PAGED>), dim3(pl.grid), dim3(NW * kWave),
                     0, st, reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k_act),
                     reinterpret_cast<const T*>(v_act), idx, items, meta, s.H, s.B, s.Bk, s.L, s.nKB, s.nQB, pl.heads_per_phase,
                     scale_log2, o_sp, static_cast<PartT*>(po), pml, pg);
}

template <typename T, int D, bool PAGED>
void dispatch_attn(const Dims& s, const SparsePlan& pl, const void* q, const void* k_act, const void* v_act,
                   const int32_t* idx, const int4* items, const int* meta, float* o_sp,
                   void* po, float* pml, const PagedKV<PAGED>& pg, hipStream_t st) {
  const int QT = s.B / 16;
  const int nw = (QT + 1) / 2;  // at most two 16-row query tiles per wave
  const int qpw = (QT + nw - 1) / nw;
#define HSA_ATTN_CASE(NW_, QPW_) \
  if (nw == NW_ && qpw == QPW_) return launch_attn<T, D, NW_, QPW_, PAGED>(s, pl, q, k_act, v_act, idx, items, meta, o_sp, po, pml, pg, st);
  HSA_ATTN_CASE(1, 1)
  HSA_ATTN_CASE(1, 2)
  HSA_ATTN_CASE(2, 2)
  HSA_ATTN_CASE(3, 2)
  HSA_ATTN_CASE(4, 2)
  HSA_ATTN_CASE(5, 2)
  HSA_ATTN_CASE(6, 2)
#undef HSA_ATTN_CASE
}

}  // namespace
}  // namespace hsa

namespace hsa {
namespace {

template <int D, typename PartT>
hsa_rc launch_combine(const Dims& s, const int2* rowinfo, const void* po, const float* pml, float* o_sp,
                      size_t comb_lds, hipStream_t st) {
  auto comb = sparse_combine_kernel<D, PartT>;
  if (comb_lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(comb), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)comb_lds) != hipSuccess)
    return HSA_ERR_HIP;
  hipLaunchKernelGGL(comb, dim3(s.rows * kCombParts), dim3(kCombThreads), comb_lds, st, rowinfo,
                     static_cast<const PartT*>(po), pml, s.H, s.B, s.nQB, o_sp);
  return HSA_OK;
}

template <bool PAGED>
hsa_rc sparse_entry(const Dims& s, const void* q, const void* k_act, const void* v_act, const int32_t* blk_count,
                    const int32_t* blk_idx, float* o_sp, void* ws, size_t ws_bytes, hsa_stream stream,
                    hsa_event ev_begin, hsa_event ev_end, const PagedKV<PAGED>& pg) {
  const WsLayout w = ws_layout(s, 1);
  if (!ws || ws_bytes < w.sp_end) return HSA_ERR_WORKSPACE;
  const SparsePlan pl = sparse_plan(s);
  if (pl.max_segs > kMaxPlanSegs) return HSA_ERR_BAD_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  int4* items = reinterpret_cast<int4*>(wsb + w.sp_items);
  int2* rowinfo = reinterpret_cast<int2*>(wsb + w.sp_rowinfo);
  int* meta = reinterpret_cast<int*>(wsb + w.sp_meta);
  void* po = wsb + w.sp_part_o;
  float* pml = reinterpret_cast<float*>(wsb + w.sp_part_ml);
  const int gps = s.bf16 ? 2 : 1;
  hipLaunchKernelGGL(sparse_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, blk_count, blk_idx, s.rows, s.nQB,
                     s.nKB, pl.granules_per_block, gps, pl.seg_granules, pl.bucket_shift, pl.heads_per_phase, items,
                     rowinfo, meta);
  if (ev_begin && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return HSA_ERR_HIP;
  if (s.bf16) {
    if (s.d == 128) dispatch_attn<bf16_t, 128, PAGED>(s, pl, q, k_act, v_act, blk_idx, items, meta, o_sp, po, pml, pg, st);
    else dispatch_attn<bf16_t, 64, PAGED>(s, pl, q, k_act, v_act, blk_idx, items, meta, o_sp, po, pml, pg, st);
  } else {
    if (s.d == 128) dispatch_attn<float, 128, PAGED>(s, pl, q, k_act, v_act, blk_idx, items, meta, o_sp, po, pml, pg, st);
    else dispatch_attn<float, 64, PAGED>(s, pl, q, k_act, v_act, blk_idx, items, meta, o_sp, po, pml, pg, st);
  }
  if (ev_end && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_end), st) != hipSuccess) return HSA_ERR_HIP;
  const size_t comb_lds = (size_t)pl.max_segs * s.B * sizeof(float2);
  hsa_rc rc;
  if (s.bf16) {
    if (s.d == 128) rc = launch_combine<128, _Float16>(s, rowinfo, po, pml, o_sp, comb_lds, st);
    else rc = launch_combine<64, _Float16>(s, rowinfo, po, pml, o_sp, comb_lds, st);
  } else {
    if (s.d == 128) rc = launch_combine<128, float>(s, rowinfo, po, pml, o_sp, comb_lds, st);
    else rc = launch_combine<64, float>(s, rowinfo, po, pml, o_sp, comb_lds, st);
  }
  if (rc != HSA_OK) return rc;
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_sparse_attn_timed(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                                        const int32_t* blk_count, const int32_t* blk_idx, float* o_sp, void* ws,
                                        size_t ws_bytes, hsa_stream stream, hsa_event ev_begin, hsa_event ev_end) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !k_act || !v_act || !blk_count || !blk_idx || !o_sp) return HSA_ERR_NULL_ARG;
  return sparse_entry<false>(s, q, k_act, v_act, blk_count, blk_idx, o_sp, ws, ws_bytes, stream, ev_begin, ev_end,
                             PagedKV<false>{});
}

extern "C" hsa_rc hsa_sparse_attn_paged(const hsa_geom* geom, const void* q, const void* const* page_k,
                                        const void* const* page_v, int32_t n_pages, const int32_t* sel_pages,
                                        const int32_t* blk_count, const int32_t* blk_idx, float* o_sp, void* ws,
                                        size_t ws_bytes, hsa_stream stream, hsa_event ev_begin, hsa_event ev_end) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !page_k || !page_v || !sel_pages || !blk_count || !blk_idx || !o_sp) return HSA_ERR_NULL_ARG;
  if (n_pages < 1 || n_pages > HSA_MAX_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
  PagedKV<true> pg;
  for (int j = 0; j < kMaxPages; ++j) pg.pk.p[j] = pg.pv.p[j] = nullptr;
  for (int j = 0; j < n_pages; ++j) {
    if (!page_k[j] || !page_v[j]) return HSA_ERR_NULL_ARG;
    pg.pk.p[j] = page_k[j];
    pg.pv.p[j] = page_v[j];
  }
  pg.sel = sel_pages;
  pg.n_pages = n_pages;
  pg.Lp = s.Lp;
  return sparse_entry<true>(s, q, nullptr, nullptr, blk_count, blk_idx, o_sp, ws, ws_bytes, stream, ev_begin, ev_end,
                            pg);
}

extern "C" hsa_rc hsa_sparse_attn_paged_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                               const void* const* page_v_table, int32_t n_pages,
                                               const int32_t* sel_pages, const int32_t* blk_count,
                                               const int32_t* blk_idx, float* o_sp, void* ws, size_t ws_bytes,
                                               hsa_stream stream, hsa_event ev_begin, hsa_event ev_end) {
  using namespace hsa;
  Dims s;
  hsa_rc rc = derive(geom, &s);
  if (rc != HSA_OK) return rc;
  if (!q || !page_k_table || !page_v_table || !sel_pages || !blk_count || !blk_idx || !o_sp) return HSA_ERR_NULL_ARG;
  if (n_pages < 1 || n_pages > HSA_MAX_BANK_PAGES || s.Kp > n_pages) return HSA_ERR_BAD_PARAM;
  PagedKV<true> pg;
  for (int k = 0; k < kMaxPages; ++k) pg.pk.p[k] = pg.pv.p[k] = nullptr;
  pg.dk = page_k_table;
  pg.dv = page_v_table;
  pg.sel = sel_pages;
  pg.n_pages = n_pages;
  pg.Lp = s.Lp;
  return sparse_entry<true>(s, q, nullptr, nullptr, blk_count, blk_idx, o_sp, ws, ws_bytes, stream, ev_begin, ev_end,
                            pg);
}

extern "C" hsa_rc hsa_sparse_attn(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                                  const int32_t* blk_count, const int32_t* blk_idx, float* o_sp, void* ws,
                                  size_t ws_bytes, hsa_stream stream) {
  return hsa_sparse_attn_timed(geom, q, k_act, v_act, blk_count, blk_idx, o_sp, ws, ws_bytes, stream, nullptr,
                               nullptr);
}
