// Device-side building blocks shared by the HIP kernels of the quantized MoE block.
//
// Packed tile format (written by pack.cpp, read by every kernel):
//   4-bit matrix [N x K]: tiles of 64 rows x 64 columns (one quantisation group),
//   tile (nb, g) at byte (nb * K/64 + g) * 2304:
//     [0, 2048)    codes: half h (columns g*64 + h*32 .. +32) of row r at h*1024 + r*16,
//                  4 words; word j holds columns c0 = h*32 + 8j .. c0+7, where
//                  column c0 + 2t sits in bits [4t, 4t+4) and c0 + 2t + 1 in
//                  bits [16 + 4t, 16 + 4t + 4)  (t = 0..3)
//     [2048, 2304) (s, b) of row r at 2048 + r*4: s in the low half, b in the high
//                  half, bf16 bit patterns
//   8-bit matrix [N x K]: tile (nb, g) at (nb * K/64 + g) * 4352:
//     [0, 4096)    codes: quarter c (columns g*64 + c*16 .. +16) of row r at c*1024 + r*16
//     [4096, 4352) (s, b) as above
// So a wavefront whose lane r owns row r reads 1 KiB contiguous per 16-byte load,
// and one 32-bit code word masked with 0x000F000F after a shift of 4t gives the
// bf16 pair (128 + q[c0+2t], 128 + q[c0+2t+1]) once 0x43004300 is OR-ed in
// (0x4300 | q is the bf16 value 128 + q for q < 16).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// a compile-time int as a value (selects template code from a runtime branch)
template <int I>
using ic = std::integral_constant<int, I>;

constexpr int kGroup = 64;
constexpr int kTile4 = 2304;
constexpr int kTile4Codes = 2048;
constexpr int kTile8 = 4352;
constexpr int kTile8Codes = 4096;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// bf16 pair (128 + q[c0 + 2t], 128 + q[c0 + 2t + 1]) of a packed 4-bit code word
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int t) {
  return ((w >> (4 * t)) & 0x000F000Fu) | 0x43004300u;
}

// power of two that brings a row maximum m (> 0) into [2^14, 2^15); 1 for m == 0
__device__ __forceinline__ float row_scale(float m) {
  if (!(m > 0.0f)) return 1.0f;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;  // floor(log2 m) for normal m
  return ldexpf(1.0f, min(14 - e, 126));
}

__device__ __forceinline__ uint16_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// nib_pair with its two constants held in registers (the mask in an SGPR, the exponent
// bits in a VGPR): a pair is then one shift and one v_and_or_b32, where literal
// operands cost a shift, an and and an or.
// kExpo: the exponent bits OR-ed into both halves (0x43004300: bf16 128 + q; 0x64006400:
// fp16 1024 + q).
template <uint32_t kExpo = 0x43004300u>
struct NibKT {
  uint32_t mask, expo;
  __device__ __forceinline__ NibKT() {
    asm("s_mov_b32 %0, 0xf000f" : "=s"(mask));
    asm("v_mov_b32 %0, %1" : "=v"(expo) : "n"(kExpo));
  }
  __device__ __forceinline__ uint32_t pair(uint32_t w, int t) const { return ((w >> (4 * t)) & mask) | expo; }
};
using NibK = NibKT<>;

// tanh form of GELU (Hendrycks & Gimpel), fp32: 0.5 z (1 + tanh u) with
// u = sqrt(2/pi) (z + 0.044715 z^3), evaluated as z / (1 + exp(-2u)) (the same
// function: (1 + tanh u) / 2 is the logistic function of 2u) with the hardware
// exp2 and a division; z -> -inf gives z / inf = 0 and z -> +inf gives z.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float t = exp2f(c2 * (z + 0.044715f * z * z * z));
  return z / (1.0f + t);
}

// Sum over the 64 lanes of a wavefront, returned to every lane. DPP row operations
// (pair and quad swaps, half-row and row mirrors, then the row broadcasts of lanes
// 15 and 31) leave the total in lane 63, which is read out: a few VALU operations
// instead of a chain of LDS-routed shuffles.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask,
                                                                   0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);  // row_mirror: every lane of a row holds the row's sum
  v = dpp_add<0x142, 0xa>(v);  // row_bcast15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast31 into rows 2 and 3: lane 63 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over the 16 lanes of each DPP row (lanes 16q .. 16q + 15), returned to every
// lane of the row: the first four steps of wave_sum with fmaxf in place of add (so a
// NaN is skipped, as fmaxf does).
template <int kCtrl>
__device__ __forceinline__ float dpp_fmax(float v) {
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf,
                                                                        0xf, false)));
}
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_fmax<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_fmax<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_fmax<0x141>(v);  // row_half_mirror
  return dpp_fmax<0x140>(v);  // row_mirror
}
// fmaxf over the 64 lanes of a wavefront, the same value in every lane (a NaN is
// skipped, as fmaxf does): the four row maxima read from lanes 0, 16, 32 and 48
__device__ __forceinline__ float wave_fmax(float v) {
  v = row16_max(v);
  auto lane_f = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return fmaxf(fmaxf(lane_f(0), lane_f(16)), fmaxf(lane_f(32), lane_f(48)));
}

// Maximum over the 64 lanes of a wavefront (unsigned), returned to every lane: the
// DPP steps of wave_sum with max in place of add (rows outside a step's row mask keep
// their value: the moved-in 0 is the identity of max on unsigned values).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xf, false);
  return v > o ? v : o;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max<0xB1, 0xf>(v);
  v = dpp_max<0x4E, 0xf>(v);
  v = dpp_max<0x141, 0xf>(v);
  v = dpp_max<0x140, 0xf>(v);
  v = dpp_max<0x142, 0xa>(v);
  v = dpp_max<0x143, 0xc>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// lane `l` (wave-uniform) of a double across the wavefront, without an LDS round trip
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// a wave-uniform pointer moved to scalar registers (the compiler cannot always prove
// uniformity, e.g. of a pointer loaded from memory through a uniform index)
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Raw buffer loads: a scalar resource (base, size in bytes) plus a per-lane 32-bit
// offset and a scalar offset, so a loop that walks a uniform stride adds nothing per
// lane. Loads past `bytes` return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t bld4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ u32x4_t bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ldg4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// Cross-workgroup hand-off inside one kernel without cache flushes. The 8 XCDs
// of the chip each have their own L2, which is not coherent with the others for
// ordinary accesses; an agent-scope fence therefore writes back and invalidates
// the whole local L2 (buffer_wbl2 / buffer_inv), and with hundreds of
// workgroups fencing those serialise. Instead, data handed to another
// workgroup is stored and loaded with agent-scope relaxed atomics (sc1: write
// through to / read from the coherence point), the producer waits for its
// stores to complete (vmcnt(0)) before it bumps the arrival counter, and the
// consumer that sees the final count reads with sc1 loads.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t arrive(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// device error word (bit flags, see moe.h); the library is one translation unit
__device__ uint32_t g_moe_device_error = 0;

__device__ __forceinline__ void flag_device_error(uint32_t bits) { atomicOr(&g_moe_device_error, bits); }

// blob of routed expert `e` through the slot table; nullptr (and the error flag) if the id or
// the table entry is out of range. With skip_ok, an entry MOE_SLOT_SKIP gives nullptr
// without the flag (an expert left out of a prefill pass on purpose).
constexpr uint32_t kSlotSkip = 0xFFFFFFFFu;
__device__ __forceinline__ const uint8_t* expert_blob(const uint8_t* pool, uint64_t stride, uint64_t n_blobs,
                                                      const uint32_t* slot_table, int e, int n_experts,
                                                      bool skip_ok = false) {
  if (e < 0 || e >= n_experts) {
    flag_device_error(2u);
    return nullptr;
  }
  uint32_t b = slot_table[e];
  if (skip_ok && b == kSlotSkip) return nullptr;
  if ((uint64_t)b >= n_blobs) {
    flag_device_error(1u);
    return nullptr;
  }
  return pool + (uint64_t)b * stride;
}

// bytes of a packed 4-bit matrix [rows x cols]
__host__ __device__ __forceinline__ uint64_t m4_bytes(int rows, int cols) {
  return (uint64_t)(rows / 64) * (uint64_t)(cols / 64) * kTile4;
}

}  // namespace qmoe
