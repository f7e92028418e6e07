// Device helpers shared by the HIP sources: lane exchanges inside a 64-lane wave and
// direct global -> LDS copies with explicit waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {
namespace {

// The value of lane `lane ^ m` (m a power of two below 64).  Inside a 16-lane row the
// exchange is a DPP lane move (quad permutes for 1 and 2, a shift left or right by 4, a
// rotation by 8), with no round trip through the LDS crossbar; 16 and 32 cross rows with a
// bpermute.  m is a constant after unrolling, so the branches fold.
__device__ __forceinline__ float lane_xor(float x, int m, int lane) {
  const int v = __builtin_bit_cast(int, x);
  if (m == 1) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  if (m == 2) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  if (m == 4) {
    const int from_above = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4, lane i + 4
    const int from_below = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4, lane i - 4
    return __builtin_bit_cast(float, (lane & 4) ? from_below : from_above);
  }
  if (m == 8) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  return __shfl_xor(x, m);
}

// A DPP lane move of x within each 16-lane row (CTRL: the DPP control, e.g. 0x128 row_ror:8).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// The pair {v[l], v[l ^ 16]} (or l ^ 32) in some order, with the row (half) swaps of
// gfx950: plain vector instructions, no round trip through the LDS crossbar.  Reductions
// (max, sum) over the pair do not depend on the order.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_rows(float v) {  // max over lanes l, l^16, l^32, l^48
  float a, b;
  pair16(v, a, b);
  pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_rows(float v) {  // sum over lanes l, l^16, l^32, l^48
  float a, b;
  pair16(v, a, b);
  pair32(a + b, a, b);
  return a + b;
}

// Direct global -> LDS copies: every lane reads BYTES bytes and the data lands in LDS at
// lds_base + lane * stride (lds_base is wave-uniform, passed in M0), where the stride is
// BYTES for 4- and 16-byte copies and 16 for 12-byte copies (the fourth dword of each lane
// is left untouched).  They count in vmcnt
// like ordinary loads but leave no register results, so a deep prefetch ring costs no
// VGPRs.  Written as inline assembly: the compiler would otherwise make every later LDS
// read wait for all of them.  The caller waits with vm_wait before reading the data.
// STREAM marks data read once (the cache stream): the non-temporal policy, which on this
// chip lifts a pure read stream from about 6.2 to 7.0 TB/s.
template <int BYTES, bool STREAM>
__device__ __forceinline__ void lds_dma(uint32_t lds_base, const void* sbase, uint32_t voff) {
  if (BYTES == 16) {
    if (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
  } else if (BYTES == 12) {
    if (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx3 %1, %2 nt" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx3 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
  } else if (BYTES == 4) {
    if (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
                   : "memory", "m0");
  } else {
    static_assert(BYTES == 4 || BYTES == 12 || BYTES == 16, "whole-lane copies of 4, 12 or 16 bytes");
  }
}
template <int BYTES, bool STREAM>
__device__ __forceinline__ void lds_dma_addr(uint32_t lds_base, const void* addr) {
  if (BYTES == 16) {
    if (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_base), "v"(addr) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(addr) : "memory", "m0");
  } else if (BYTES == 4) {
    if (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off nt" ::"s"(lds_base), "v"(addr) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(addr) : "memory", "m0");
  } else {
    static_assert(BYTES == 4 || BYTES == 16, "whole-lane copies of 4 or 16 bytes");
  }
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until every LDS access of this wave is complete.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------------------
// Quaternions (real, i, j, k): the IsoQuant block rotation v -> q_L v conj(q_R).
struct Quat {
  float w, x, y, z;
};
__device__ __forceinline__ Quat qmul(Quat a, Quat b) {
  return {a.w * b.w - a.x * b.x - a.y * b.y - a.z * b.z, a.w * b.x + a.x * b.w + a.y * b.z - a.z * b.y,
          a.w * b.y - a.x * b.z + a.y * b.w + a.z * b.x, a.w * b.z + a.x * b.y - a.y * b.x + a.z * b.w};
}
__device__ __forceinline__ Quat qconj(Quat a) { return {a.w, -a.x, -a.y, -a.z}; }
__device__ __forceinline__ Quat qload(const float* p) {
  const float4 v = *(const float4*)p;
  return {v.x, v.y, v.z, v.w};
}

// Rotation of nh head vectors held in LDS (buf[nh][128]) by the whole workgroup.
// Forward: signs, normalised Hadamard on every `group` block, then SO(4) if present.
// Inverse: the reverse.  Called uniformly by every thread of the block.
template <bool FWD>
__device__ void lds_rotate(float* buf, int nh, const float* signs, const float* so4, int group) {
  const int nt = blockDim.x, tid = threadIdx.x, n = nh * 128;
  if (FWD) {
    for (int i = tid; i < n; i += nt) buf[i] *= signs[i & 127];
    __syncthreads();
  } else if (so4 != nullptr) {
    for (int p = tid; p < nh * 32; p += nt) {
      float* v = buf + (p >> 5) * 128 + 4 * (p & 31);
      const Quat l = qload(so4 + 8 * (p & 31)), r = qload(so4 + 8 * (p & 31) + 4);
      const Quat o = qmul(qmul(qconj(l), Quat{v[0], v[1], v[2], v[3]}), r);
      v[0] = o.w; v[1] = o.x; v[2] = o.y; v[3] = o.z;
    }
    __syncthreads();
  }
  for (int s = 1; s < group; s <<= 1) {
    for (int p = tid; p < nh * 64; p += nt) {
      const int j = p & 63;
      const int i0 = (p >> 6) * 128 + (j / s) * 2 * s + (j % s);
      const float x0 = buf[i0], x1 = buf[i0 + s];
      buf[i0] = x0 + x1;
      buf[i0 + s] = x0 - x1;
    }
    __syncthreads();
  }
  const float hs = group == 32 ? 0.17677669529663688f : 0.088388347648318440f;
  if (FWD) {
    for (int i = tid; i < n; i += nt) buf[i] *= hs;
    __syncthreads();
    if (so4 != nullptr) {
      for (int p = tid; p < nh * 32; p += nt) {
        float* v = buf + (p >> 5) * 128 + 4 * (p & 31);
        const Quat l = qload(so4 + 8 * (p & 31)), r = qload(so4 + 8 * (p & 31) + 4);
        const Quat o = qmul(qmul(l, Quat{v[0], v[1], v[2], v[3]}), qconj(r));
        v[0] = o.w; v[1] = o.x; v[2] = o.y; v[3] = o.z;
      }
      __syncthreads();
    }
  } else {
    for (int i = tid; i < n; i += nt) buf[i] *= hs * signs[i & 127];
    __syncthreads();
  }
}



}  // namespace
}  // namespace tq
