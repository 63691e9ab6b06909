// Device-side helpers shared by the HSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsa_attn.h"

namespace hsa {

typedef uint16_t bf16_t;  // storage of a bfloat16 value
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxPages = HSA_MAX_PAGES;

// 1 KB of zeros in device memory: the source of the 16-byte lanes of direct
// global->LDS loads whose contraction elements must be zero (each lane reads
// kZeroPage[lane]).
__device__ const uint4 kZeroPage[64] = {};

// Page pointer tables: by value as launch arguments (up to HSA_MAX_PAGES
// pages), or a device array of pointers (up to HSA_MAX_BANK_PAGES).  Kernels
// take either through at(j).
struct PageTable {
  const void* p[kMaxPages];
  __device__ __forceinline__ const void* at(int j) const { return p[j]; }
};
struct DevPageTable {
  const void* const* p;
  __device__ __forceinline__ const void* at(int j) const { return p[j]; }
};

// Keys and values read in place from laid-out pages (PAGED kernels): page j
// holds K as [H][Lp][d] and V as [H][Lp/16][d][16] (the active buffer's
// layouts over one page), and active key t is token t % Lp of page
// sel[t / Lp].  The page pointers come from a table passed by value (pk, pv)
// or, for banks larger than one launch argument holds, from tables in device
// memory (dk, dv, used when non-NULL); a NULL page there reads as zeros.  The
// unpaged form carries nothing.
template <bool PAGED> struct PagedKV {
  static constexpr int Lp = 0;
};
template <> struct PagedKV<true> {
  PageTable pk, pv;
  const void* const* dk = nullptr;
  const void* const* dv = nullptr;
  const int32_t* sel;
  int n_pages, Lp;
  __device__ __forceinline__ const void* kpage(int j) const { return dk ? dk[j] : pk.p[j]; }
  __device__ __forceinline__ const void* vpage(int j) const { return dv ? dv[j] : pv.p[j]; }
};

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Elements of T in one 16-byte chunk.
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

// Unpack a 16-byte chunk of T into floats.
template <typename T> __device__ __forceinline__ void unpack16(const uint4& c, float* out);
template <> __device__ __forceinline__ void unpack16<float>(const uint4& c, float* out) {
  out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
  out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
}
template <> __device__ __forceinline__ void unpack16<bf16_t>(const uint4& c, float* out) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Pack floats into a 16-byte chunk of T.
template <typename T> __device__ __forceinline__ uint4 pack16(const float* in);
template <> __device__ __forceinline__ uint4 pack16<float>(const float* in) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]), __float_as_uint(in[3]));
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
template <> __device__ __forceinline__ uint4 pack16<bf16_t>(const float* in) {
  return make_uint4(pack2_bf16(in[0], in[1]), pack2_bf16(in[2], in[3]), pack2_bf16(in[4], in[5]), pack2_bf16(in[6], in[7]));
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// 16-byte load of data read once (a stream): the non-temporal hint keeps it
// from displacing cached data.  Measured: page scoring 5.2 -> 5.7 TB/s, the
// page gather 5.8 -> 5.9 TB/s.  Data written shortly before (the merge of
// split rows) reads slower with it.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// 16-byte load that is always issued, zeroed where `ok` is false.  The
// address must be valid in every lane (callers clamp it); a load under a
// per-lane condition is otherwise split into dword loads, each waited for.
__device__ __forceinline__ uint4 ld16_masked(const void* p, bool ok) {
  const uint4 v = ld16(p);
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// 16x16 matrix-core step.  Lane l = 16*g + c (g = l/16 in 0..3, c = l%16)
// supplies one 16-byte chunk of A row c and one of B column c; both chunks
// hold the contraction elements of "slot g".  Any assignment of contraction
// indices to (g, element) works as long as A and B use the same one, because
// the product sums over all of them.  The result is the standard 16x16 layout:
// lane (g, c) holds C[4g + i][c] in acc[i].
//   bf16: contraction 32 per step (8 per lane), v_mfma_f32_16x16x32_bf16.
//   f32 : contraction 16 per step (4 per lane), four v_mfma_f32_16x16x4_f32,
//         instruction j taking element j of every lane's chunk.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int K = 32;
  __device__ __forceinline__ static void run(f32x4& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int K = 16;
  __device__ __forceinline__ static void run(f32x4& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Row permutation inside one contraction group of a product whose result is
// fed back as the B operand of a second product (S^T -> P^T).  For bf16 the
// second product contracts 32 keys per step, covering two 16-row result
// tiles kt = 0, 1.  Loading result-tile kt row c from source row
// perm_row(kt, c) = 8*(c/4) + 4*kt + c%4 makes lane (g, q) end up holding
// source rows 8g .. 8g+7, i.e. one contiguous chunk of the second product's
// operand.  For f32 (one 16-row tile per step) the identity does the same.
template <typename T> __device__ __forceinline__ int perm_row(int kt, int c);
template <> __device__ __forceinline__ int perm_row<bf16_t>(int kt, int c) { return 8 * (c >> 2) + 4 * kt + (c & 3); }
template <> __device__ __forceinline__ int perm_row<float>(int kt, int c) { return c; }

// Pack the probabilities a lane holds for one contraction step into the B chunk.
template <typename T> __device__ __forceinline__ uint4 pack_p(const f32x4* p);
template <> __device__ __forceinline__ uint4 pack_p<bf16_t>(const f32x4* p) {
  float t[8] = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
  return pack16<bf16_t>(t);
}
template <> __device__ __forceinline__ uint4 pack_p<float>(const f32x4* p) {
  return make_uint4(__float_as_uint(p[0][0]), __float_as_uint(p[0][1]), __float_as_uint(p[0][2]), __float_as_uint(p[0][3]));
}

// Cross-lane reductions over the four lanes (g = 0..3) that share c = l%16,
// with the gfx950 row swaps (plain VALU, no LDS round trip).  With both
// operands equal, v_permlane16_swap returns the rows exchanged in pairs
// (0,1) / (2,3) across its two results, v_permlane32_swap in pairs (0,2) /
// (1,3); combining its two results reduces over lanes l and l^16 (l^32) in
// every lane, in the same order in all four lanes.
// Maximum of two values that are never NaN, as one v_max_f32 (the plain
// comparison costs a compare and a select, fmaxf adds canonicalizations).
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max4g(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nn(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum4g(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Direct global->LDS loads: one wave instruction moves 64 lanes x 16 bytes
// into 1 KB of contiguous LDS (lane l -> bytes 16l..16l+15 of the wave base).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void load_lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// wait until this wave's direct-to-LDS (and other vector memory) loads have landed
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for the staging ring: this wave's LDS reads are done and
// at most N of its direct-to-LDS loads are still in flight, then all waves
// meet.  (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14.)  The empty asm statements keep the compiler from moving
// LDS accesses across the barrier, which __builtin_amdgcn_s_barrier alone
// does not; unlike __syncthreads they do not force every load to land.
template <int N> __device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Word 3 of a buffer resource for raw (untyped) buffer loads on gfx9-family
// chips such as gfx950: 32-bit data format, no swizzle, no stride.  Loads
// past num_records read zeros.
constexpr int kBufferRsrcWord3 = 0x00020000;

// One direct buffer->LDS load of 16 bytes per lane: the resource spans
// [base, base + bytes), the lane reads at byte voffset + soffset (soffset
// uniform) and lands at lds_wave_base + 16 * lane.  The address of a lane
// takes one 32-bit register instead of a 64-bit pair.  (Kept out of lambdas:
// called from one, the builtin made the compiler drop the kernel's host stub.)
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, void* lds_wave_base, int voffset,
                                                  int soffset) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voffset, soffset, 0, 0);
}

// Swizzle of row-major operand tiles in LDS: the 16-byte chunk c of row rho
// sits in slot c ^ kswz(rho).  A matrix-core A operand is read as 16 rows
// (perm_row(kt, c) for lanes c = 0..15, see above) at one chunk index; the
// swizzle sends those 16 reads to distinct banks.
template <typename T> __device__ __forceinline__ int kswz(int rho, int cpr);
template <> __device__ __forceinline__ int kswz<bf16_t>(int rho, int cpr) {
  return ((rho & 3) | (((rho >> 3) & 3) << 2)) & (cpr - 1);
}
template <> __device__ __forceinline__ int kswz<float>(int rho, int cpr) { return rho & 15 & (cpr - 1); }

// 2^x with the hardware instruction (no range fix-ups): used for softmax
// weights whose arguments are <= 8 here; results below the float range flush
// to 0, which is what the softmax wants.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The 8 XCDs of an MI355X receive consecutive workgroup ids round-robin.
// Remapping blockIdx so that each XCD walks one contiguous range of work
// items keeps the items an XCD runs together (same head, same K/V) in that
// XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = ceil_div(n, 8);
  const int x = bid & 7, k = bid >> 3;
  const int item = x * per + k;
  return (k < per && item < n) ? item : -1;
}

}  // namespace hsa
