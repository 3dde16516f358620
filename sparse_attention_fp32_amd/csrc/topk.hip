// a4: pool top-k with lowest-id tie-breaking, emitted in ascending pool id.
//
// One 1024-thread workgroup per score row.  Each thread keeps a contiguous run
// of E ids as order-preserving integer keys in registers (a finite float maps
// to an unsigned key that sorts like the float; non-candidates are key 0 and
// never counted).  A byte-wise radix select over LDS histograms finds the
// threshold key T of the k_eff-th best candidate (stopping early once the
// threshold bin is taken whole); then every key above T is kept, and among the
// keys equal to T the lowest ids, via a block prefix sum in id order.  A second
// prefix sum writes the kept ids ascending.  No floating-point comparison is
// involved, so the result depends only on the score bits.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int s = lane < kWaves ? s_wave[lane] : 0;
    const int own = s;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const int y = __shfl_up(s, o, kWave);
      if (lane >= o) s += y;
    }
    if (lane < kWaves) s_wave[kWaves + lane] = s - own;  // exclusive wave offsets
    if (lane == kWaves - 1) s_wave[2 * kWaves] = s;
  }
  __syncthreads();
  const int res = x - v + s_wave[kWaves + wv];
  *total = s_wave[2 * kWaves];
  __syncthreads();
  return res;
}

template <int E>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const uint8_t* __restrict__ cand,
                                                        int pstride, int select_k,
                                                        int32_t* __restrict__ sel) {
  __shared__ int hist[256];
  __shared__ int s_wave[2 * kWaves + 1];
  __shared__ int s_bin, s_above, s_binc;
  const int q = blockIdx.x, t = threadIdx.x;
  const float* srow = scores + (int64_t)q * pstride;
  const uint8_t* crow = cand + (int64_t)q * pstride;
  int32_t* out = sel + (int64_t)q * select_k;

  // all loads issued together (ids clamped into the row), then masked
  uint32_t key[E];
  float sv[E];
  uint8_t cv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int id = min(t * E + e, pstride - 1);
    sv[e] = srow[id];
    cv[e] = crow[id];
  }
  int nc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = t * E + e < pstride && cv[e] != 0;
    key[e] = c ? float_order_key(sv[e]) : 0u;
    nc += c;
  }
  int ncand;
  (void)block_exclusive_scan(nc, s_wave, &ncand);
  const int k_eff = min(select_k, ncand);
  if (k_eff == 0) {
    for (int i = t; i < select_k; i += kThreads) out[i] = -1;
    return;
  }

  uint32_t prefix = 0u, mask = 0u;
  int krem = k_eff;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (t < 256) hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1);
    __syncthreads();
    if (t < 64) {
      int h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = hist[4 * t + j];
      const int sl = h[0] + h[1] + h[2] + h[3];
      int x = sl;  // inclusive suffix sum over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(x, o, kWave);
        if (t + o < 64) x += y;
      }
      int above = x - sl;  // keys in higher bins of higher lanes
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < krem && krem <= above + h[j]) {
          s_bin = 4 * t + j;
          s_above = above;
          s_binc = h[j];
        }
        above += h[j];
      }
    }
    __syncthreads();
    const int b = s_bin, bc = s_binc;
    krem -= s_above;
    prefix |= (uint32_t)b << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
    if (bc == krem) break;  // the whole threshold bin is taken
  }

  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] == 0u) continue;
    const uint32_t km = key[e] & mask;
    n_gt += km > prefix;
    n_eq += km == prefix;
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, s_wave, &tot);
  const int take_eq = max(0, min(n_eq, krem - eq_before));
  const int pos0 = block_exclusive_scan(n_gt + take_eq, s_wave, &tot);
  int pos = pos0, eq_taken = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] == 0u) continue;
    const uint32_t km = key[e] & mask;
    bool take = km > prefix;
    if (km == prefix) take = eq_taken++ < take_eq;
    if (take && pos < k_eff) out[pos++] = t * E + e;
  }
  for (int i = k_eff + t; i < select_k; i += kThreads) out[i] = -1;
}

}  // namespace

DSA_EXPORT size_t dsa_topk_pools_workspace_size(int Q, int pstride, int select_k) {
  (void)Q;
  (void)pstride;
  (void)select_k;
  return 0;
}

DSA_EXPORT dsa_status dsa_topk_pools(const float* scores, const uint8_t* cand, int Q, int pstride,
                                     int select_k, int32_t* sel, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: select_k=%d < 1", select_k);
  DSA_REQUIRE(pstride >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: pstride=%d < 1", pstride);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_topk_pools: Q=%d < 0", Q);
  DSA_REQUIRE(pstride <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED,
              "dsa_topk_pools: pstride=%d above %d", pstride, DSA_MAX_TOPK_ROW);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(scores && cand && sel, DSA_ERR_INVALID_ARG, "dsa_topk_pools: NULL tensor pointer");
  const int need = (pstride + kThreads - 1) / kThreads;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] topk_pools Q=%d pstride=%d select_k=%d E=%d\n", Q, pstride, select_k,
            need);
#define DSA_LAUNCH_TK(E) \
  topk_kernel<E><<<Q, kThreads, 0, stream>>>(scores, cand, pstride, select_k, sel)
  if (need <= 1) DSA_LAUNCH_TK(1);
  else if (need <= 2) DSA_LAUNCH_TK(2);
  else if (need <= 4) DSA_LAUNCH_TK(4);
  else if (need <= 8) DSA_LAUNCH_TK(8);
  else DSA_LAUNCH_TK(16);
#undef DSA_LAUNCH_TK
  return dsa::check_launch("dsa_topk_pools");
}
