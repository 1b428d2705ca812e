// Wave-level building blocks shared by the kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {
namespace wave {

constexpr int kWave = 64;

// wave reductions and scans with DPP lane moves (quad permutes, row shifts
// and mirrors, the row broadcasts of this ISA family): six VALU steps
// instead of a chain of LDS-routed shuffles.  Reductions leave the result in
// lane 63 and broadcast it with readlane.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// lanes that the row mask leaves out (or whose source is out of the row)
// receive `old`
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(old), __float_as_int(v)));
}
__device__ __forceinline__ float lane63_f(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppQuadXor1>(0.f, v);
  v += dpp_f<kDppQuadXor2>(0.f, v);
  v += dpp_f<kDppRowHalfMirror>(0.f, v);
  v += dpp_f<kDppRowMirror>(0.f, v);
  v += dpp_f<kDppRowBcast15, 0xA>(0.f, v);
  v += dpp_f<kDppRowBcast31, 0xC>(0.f, v);
  return lane63_f(v);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)dpp_i<kDppQuadXor1>(0, (int)v);
  v += (uint32_t)dpp_i<kDppQuadXor2>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowHalfMirror>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowMirror>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast15, 0xA>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast31, 0xC>(0, (int)v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// the maximum over each group of 8 lanes (half a DPP row), in every lane of
// the group: the quads first, then each quad against the mirrored other one
__device__ __forceinline__ float row8_max(float v) {
  const float n = -INFINITY;
  v = fmaxf(v, dpp_f<kDppQuadXor1>(n, v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(n, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(n, v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  const float n = -INFINITY;
  v = fmaxf(v, dpp_f<kDppQuadXor1>(n, v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(n, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(n, v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(n, v));
  v = fmaxf(v, dpp_f<kDppRowBcast15, 0xA>(n, v));
  v = fmaxf(v, dpp_f<kDppRowBcast31, 0xC>(n, v));
  return lane63_f(v);
}

__device__ __forceinline__ int wave_min_i(int v) {
  const int n = 0x7FFFFFFF;
  v = min(v, dpp_i<kDppQuadXor1>(n, v));
  v = min(v, dpp_i<kDppQuadXor2>(n, v));
  v = min(v, dpp_i<kDppRowHalfMirror>(n, v));
  v = min(v, dpp_i<kDppRowMirror>(n, v));
  v = min(v, dpp_i<kDppRowBcast15, 0xA>(n, v));
  v = min(v, dpp_i<kDppRowBcast31, 0xC>(n, v));
  return __builtin_amdgcn_readlane(v, 63);
}

// inclusive prefix over the lanes (Hillis-Steele inside rows of 16, then
// the row broadcasts carry the row totals forward)
__device__ __forceinline__ float wave_incl_scan_f(float v) {
  v += dpp_f<kDppRowShr1>(0.f, v);
  v += dpp_f<kDppRowShr2>(0.f, v);
  v += dpp_f<kDppRowShr4>(0.f, v);
  v += dpp_f<kDppRowShr8>(0.f, v);
  v += dpp_f<kDppRowBcast15, 0xA>(0.f, v);
  v += dpp_f<kDppRowBcast31, 0xC>(0.f, v);
  return v;
}

// maximum of an int over the wave, in every lane
__device__ __forceinline__ int wave_max_i(int v) {
  const int n = (int)0x80000000u;
  v = max(v, dpp_i<kDppQuadXor1>(n, v));
  v = max(v, dpp_i<kDppQuadXor2>(n, v));
  v = max(v, dpp_i<kDppRowHalfMirror>(n, v));
  v = max(v, dpp_i<kDppRowMirror>(n, v));
  v = max(v, dpp_i<kDppRowBcast15, 0xA>(n, v));
  v = max(v, dpp_i<kDppRowBcast31, 0xC>(n, v));
  return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace wave
}  // namespace sv
