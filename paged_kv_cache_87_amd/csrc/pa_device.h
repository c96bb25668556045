// Device helpers shared by the gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A bf16 is the high half of a binary32, so widening is a
// shift; narrowing rounds to nearest, ties to even, and keeps NaNs quiet.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// Cross-lane moves inside a 16-lane DPP row (wave64 = 4 rows).
// ---------------------------------------------------------------------------
namespace dpp {
constexpr int kRowMirror = 0x140;      // lane i of a row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141;  // lane i of each 8-lane half reads lane 7 - i
constexpr int kQuadReverse = 0x1B;     // quad_perm [3,2,1,0]: lane i of a quad reads 3 - i
constexpr int kQuadSwapPairs = 0xB1;   // quad_perm [1,0,3,2]: lane i of a quad reads i ^ 1
constexpr int row_ror(int n) { return 0x120 + n; }  // rotate within the row by n (1..15)
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------------------
// Vector loads of NW consecutive dwords (NW in {2, 4, 8}) from global memory.
// ---------------------------------------------------------------------------
template <int NW>
struct Frag {
  uint32_t w[NW];
};

template <int NW>
__device__ __forceinline__ Frag<NW> load_frag(const void* ptr) {
  Frag<NW> f;
  if constexpr (NW == 2) {
    const uint2 x = *static_cast<const uint2*>(ptr);
    f.w[0] = x.x; f.w[1] = x.y;
  } else if constexpr (NW == 4) {
    const uint4 x = *static_cast<const uint4*>(ptr);
    f.w[0] = x.x; f.w[1] = x.y; f.w[2] = x.z; f.w[3] = x.w;
  } else {
    static_assert(NW == 8, "fragment width");
    const uint4 x = static_cast<const uint4*>(ptr)[0];
    const uint4 y = static_cast<const uint4*>(ptr)[1];
    f.w[0] = x.x; f.w[1] = x.y; f.w[2] = x.z; f.w[3] = x.w;
    f.w[4] = y.x; f.w[5] = y.y; f.w[6] = y.z; f.w[7] = y.w;
  }
  return f;
}

// ---------------------------------------------------------------------------
// Buffer loads through a per-range resource descriptor.  A descriptor whose
// size is 0 turns every load through it into a zero fill that touches no
// memory, so prefetches past the end of a range can be issued unconditionally.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9-family format word

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// AUX is the instruction's cache-policy field (2 = non-temporal on gfx950).
template <int NW, int AUX = 0>
__device__ __forceinline__ Frag<NW> load_frag_buf(Rsrc r, uint32_t voff) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  Frag<NW> f;
  if constexpr (NW == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, AUX);
    f.w[0] = x[0]; f.w[1] = x[1];
  } else if constexpr (NW == 4) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX);
    f.w[0] = x[0]; f.w[1] = x[1]; f.w[2] = x[2]; f.w[3] = x[3];
  } else {
    static_assert(NW == 8, "fragment width");
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX);
    const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, AUX);
    f.w[0] = x[0]; f.w[1] = x[1]; f.w[2] = x[2]; f.w[3] = x[3];
    f.w[4] = y[0]; f.w[5] = y[1]; f.w[6] = y[2]; f.w[7] = y[3];
  }
  return f;
}

}  // namespace pa
