// The HBM read lane: a plain coalesced read, 16 bytes per lane, that sets the
// achievable streaming rate a kernel's bandwidth is compared with.
//
// stkernel pull request #290 (its measurement ledger): a bandwidth-bound
// kernel is measured against the rate of a plain streaming kernel on the same
// part -- "the lane" -- and one at 90 % of it or more counts as at the
// bandwidth floor.  The 8 TB/s figure is the part's peak; the lane is what a
// kernel can reach.
//
// Each workgroup reads one contiguous block, sixteen 16-byte loads per lane in
// flight (on this part that runs at ~6.3 TB/s, where a grid-stride loop over
// the same bytes reaches ~5.0); the data is folded into one word that is
// stored only for a value no fill produces, so no load can be dropped.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

constexpr int kLaneWG = 4096;  // workgroups (16 per compute unit)
constexpr int kLaneU = 16;     // loads per lane in flight

__global__ __launch_bounds__(256) void lane_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte words per workgroup
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t x = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (kLaneU - 1) * 256 < hi; i += kLaneU * 256) {
    uint4 v[kLaneU];
#pragma unroll
    for (int k = 0; k < kLaneU; ++k) v[k] = src[i + k * 256];
#pragma unroll
    for (int k = 0; k < kLaneU; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) *sink = x;
}

}  // namespace

DSA_EXPORT dsa_status dsa_lane_read(const void* src, size_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
  DSA_REQUIRE(bytes % 16 == 0, DSA_ERR_INVALID_ARG, "dsa_lane_read: %zu bytes, not a multiple of 16",
              bytes);
  if (bytes == 0) return DSA_OK;
  DSA_REQUIRE(src && sink, DSA_ERR_INVALID_ARG, "dsa_lane_read: NULL pointer");
  DSA_REQUIRE_ALIGNED("dsa_lane_read", src, sink);
  if (dsa::dry_run()) return DSA_OK;
  lane_read_kernel<<<kLaneWG, 256, 0, stream>>>((const uint4*)src, bytes / 16, sink);
  return dsa::check_launch("dsa_lane_read");
}
