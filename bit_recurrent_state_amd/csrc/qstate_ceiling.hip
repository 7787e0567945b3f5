// qstate_ceiling.hip — the bandwidth-ceiling kernels of include/qstate_ceiling.h:
// a streaming copy and an in-place read-modify-write over a buffer, with the
// 16-byte non-temporal accesses the decode step uses for the state.
//
// Each workgroup of 256 lanes moves tiles of 256 x UNROLL 16-byte vectors:
// all UNROLL loads of a tile are issued before the first store, so a lane
// keeps UNROLL loads in flight.  The grid is four times what the chip holds
// at once (workgroups per CU from the occupancy query) and strides over the
// tiles: later workgroups start as the first ones finish, which keeps every
// CU loaded through the end better than one resident round does.  On MI355X
// a sweep of lanes per workgroup (64..1024), unroll (1..16) and grid
// multiple (1, 2, 4, one tile per workgroup) put UNROLL = 4 with four rounds
// at the top for both kernels (about 5.9-6.0 TB/s over 4 GiB with
// non-temporal accesses).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qstate.h"
#include "qstate_ceiling.h"

namespace {

constexpr int kLanes = 256;
constexpr int kUnroll = 4;
constexpr int kRounds = 4;  // grid = kRounds x resident workgroups

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// RMW: src == dst and every word is xor-ed with pattern; else a copy.
template <bool RMW, bool NT>
__global__ __launch_bounds__(kLanes) void ceiling_kernel(const u32x4* src, u32x4* dst,
                                                          uint64_t n16, uint32_t pattern) {
  const uint64_t tile = (uint64_t)kLanes * kUnroll;
  for (uint64_t base = (uint64_t)blockIdx.x * tile; base < n16;
       base += (uint64_t)gridDim.x * tile) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = base + (uint64_t)u * kLanes + threadIdx.x;
      if (i < n16) x[u] = load16<NT>(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = base + (uint64_t)u * kLanes + threadIdx.x;
      if (i < n16) store16<NT>(dst + i, RMW ? (x[u] ^ pattern) : x[u]);
    }
  }
}

template <bool RMW, bool NT>
int launch(const void* src, void* dst, size_t bytes, uint32_t pattern, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return QSTATE_OK;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(ceiling_kernel<RMW, NT>), kLanes, 0) !=
          hipSuccess)
    return QSTATE_E_LAUNCH;
  const uint64_t tiles = (n16 + (uint64_t)kLanes * kUnroll - 1) / ((uint64_t)kLanes * kUnroll);
  const uint64_t grid =
      std::min<uint64_t>(tiles, (uint64_t)kRounds * cus * (uint64_t)std::max(per_cu, 1));
  ceiling_kernel<RMW, NT><<<(unsigned)grid, kLanes, 0, s>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16, pattern);
  return hipGetLastError() == hipSuccess ? QSTATE_OK : QSTATE_E_LAUNCH;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int qstate_ceiling_copy(const void* src, void* dst, size_t bytes, int nontemporal,
                                   void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0 ||
      (nontemporal != 0 && nontemporal != 1))
    return QSTATE_E_INVALID;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (bytes && a < b + bytes && b < a + bytes) return QSTATE_E_INVALID;  // overlap
  hipStream_t s = static_cast<hipStream_t>(stream);
  return nontemporal ? launch<false, true>(src, dst, bytes, 0, s)
                     : launch<false, false>(src, dst, bytes, 0, s);
}

extern "C" int qstate_ceiling_rmw(void* buf, size_t bytes, uint32_t pattern, int nontemporal,
                                  void* stream) {
  if (!buf || !aligned16(buf) || bytes % 16 != 0 || (nontemporal != 0 && nontemporal != 1))
    return QSTATE_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return nontemporal ? launch<true, true>(buf, buf, bytes, pattern, s)
                     : launch<true, false>(buf, buf, bytes, pattern, s);
}
