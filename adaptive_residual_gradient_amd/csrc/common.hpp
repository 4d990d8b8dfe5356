// Device helpers shared by the AdaComp kernels: streaming float4 access,
// index-word access and message constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace adacomp {


constexpr uint32_t kSentinel = 0xFFFFFFFFu;

// Non-temporal hints on the dense reads of the tile pass: residue and dW are
// read once per call, so neither should displace other data from the caches
// (a streaming probe on this chip: read-read-write 6.16 TB/s with the hints
// against 5.9 without).  The residue store's hint is a template parameter of
// the tile-pass kernels, chosen per plan (layout.hpp, kCachedResidueMaxElems).
constexpr bool kNtLoadResidue = true, kNtLoadDw = true;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming float4 access.  residue and dW are read once and the residue
// written once per call, so all three use non-temporal accesses (measured
// fastest on MI355X for this read-read-write stream).
template <bool NT>
__device__ __forceinline__ f32x4 load4(const float* p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void store4(float* p, f32x4 v) {
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = v;
}

// DPP lane moves (VALU, no LDS round trip).  Lanes without a source, and
// lanes of rows masked off, receive `old`.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROWS, 0xf, false));
}
// lane l receives lane l+1 (wave_shl:1); lane 63 receives old
__device__ __forceinline__ uint32_t from_next_lane(uint32_t old, uint32_t v) { return dpp_u32<0x130>(old, v); }
// lane l receives lane l-1 (wave_shr:1); lane 0 receives old
__device__ __forceinline__ uint32_t from_prev_lane(uint32_t old, uint32_t v) { return dpp_u32<0x138>(old, v); }

// Inclusive sum over the 64 lanes of a wavefront: row shifts 1, 2, 4, 8 scan
// within rows of 16 lanes, the row broadcasts of lanes 15/47 and then 31
// carry across rows.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
    v += dpp_u32<0x111>(0u, v);
    v += dpp_u32<0x112>(0u, v);
    v += dpp_u32<0x114>(0u, v);
    v += dpp_u32<0x118>(0u, v);
    v += dpp_u32<0x142, 0xa>(0u, v);
    v += dpp_u32<0x143, 0xc>(0u, v);
    return v;
}
// The same within each row of 16 lanes only.
__device__ __forceinline__ uint32_t row_incl_add(uint32_t v) {
    v += dpp_u32<0x111>(0u, v);
    v += dpp_u32<0x112>(0u, v);
    v += dpp_u32<0x114>(0u, v);
    v += dpp_u32<0x118>(0u, v);
    return v;
}

__device__ __forceinline__ uint64_t rup16(uint64_t x) { return (x + 15u) & ~uint64_t(15); }

__device__ __forceinline__ void put_word(uint8_t* p, uint32_t wb, uint32_t v) {
    if (wb == 1u) *p = static_cast<uint8_t>(v);
    else *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v);
}

__device__ __forceinline__ uint32_t get_word(const uint8_t* p, uint32_t wb) {
    return wb == 1u ? uint32_t(*p) : uint32_t(*reinterpret_cast<const uint16_t*>(p));
}

}  // namespace adacomp
