// a4: pool top-k with lowest-id tie-breaking, emitted in ascending pool id.
//
// One 1024-thread workgroup per score row.  Each thread keeps a contiguous run
// of E ids as order-preserving integer keys in registers (a finite float maps
// to an unsigned key that sorts like the float; non-candidates are key 0 and
// never counted), so no floating-point comparison decides the selection.
//  1. The row's largest key and the octave of every key below it (difference
//     of the top 9 key bits = sign and exponent, capped at 15) are found; the
//     octave counts are kept in registers and summed over the workgroup in a
//     fixed order -- no atomics, because nearly all scores of a row share
//     their top key bits.
//  2. Inside the octave that holds the k_eff-th best key, byte-wise radix
//     passes over per-wave LDS histograms pin the threshold key T (stopping
//     early once the threshold bin is taken whole).
//  3. Every key above T is kept and, among keys equal to T, the lowest ids,
//     via a block prefix sum in id order; a second prefix sum writes the kept
//     ids ascending.
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

// Sum of 16 per-lane counters over the wave, scattered: lane l (l % 4 == 0)
// returns the total of counter j(l) = 8*b5 + 4*b4 + 2*b3 + b2 of its lane id.
__device__ int wave_reduce_scatter16(const int (&c)[16], int lane) {
  int v8[8], v4[4], v2[2];
  {
    const bool hi = (lane >> 5) & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) v8[i] = (hi ? c[8 + i] : c[i]) + __shfl_xor(hi ? c[i] : c[8 + i], 32, kWave);
  }
  {
    const bool hi = (lane >> 4) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = (hi ? v8[4 + i] : v8[i]) + __shfl_xor(hi ? v8[i] : v8[4 + i], 16, kWave);
  }
  {
    const bool hi = (lane >> 3) & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) v2[i] = (hi ? v4[2 + i] : v4[i]) + __shfl_xor(hi ? v4[i] : v4[2 + i], 8, kWave);
  }
  const bool hi = (lane >> 2) & 1;
  int v = (hi ? v2[1] : v2[0]) + __shfl_xor(hi ? v2[0] : v2[1], 4, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 1, kWave);
  return v;
}

template <int E>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const uint8_t* __restrict__ cand,
                                                        int pstride, int select_k,
                                                        int32_t* __restrict__ sel) {
  __shared__ int hist[kWaves][256];
  __shared__ int s_tot[256];
  __shared__ int s_wave[2 * kWaves + 1];
  __shared__ uint32_t s_max[kWaves];
  __shared__ int s_oct[kWaves][16];
  __shared__ int s_bin, s_above, s_binc;
  const int q = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
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
  uint32_t kmx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = t * E + e < pstride && cv[e] != 0;
    key[e] = c ? float_order_key(sv[e]) : 0u;
    nc += c;
    kmx = max(kmx, key[e]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o, kWave));
  if (lane == 0) s_max[wv] = kmx;
  int ncand;
  (void)block_exclusive_scan(nc, s_wave, &ncand);  // its barriers also publish s_max
  const int k_eff = min(select_k, ncand);
  if (k_eff == 0) {
    for (int i = t; i < select_k; i += kThreads) out[i] = -1;
    return;
  }
  uint32_t kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) kmax = max(kmax, s_max[w]);
  const uint32_t top9 = kmax >> 23;

  // 1. octave counts (register histograms, fixed-order reduction)
  int cnt[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) cnt[b] = 0;
  uint32_t oct[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t d = min(top9 - (key[e] >> 23), 15u);
    oct[e] = key[e] ? d : 16u;
#pragma unroll
    for (int b = 0; b < 16; ++b) cnt[b] += oct[e] == (uint32_t)b;
  }
  {
    const int v = wave_reduce_scatter16(cnt, lane);
    if ((lane & 3) == 0)
      s_oct[wv][((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1)] = v;
  }
  __syncthreads();
  if (t < 64) {
    int tot = 0;
    if (t < 16)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += s_oct[w][t];
    int x = tot;  // inclusive prefix over octaves 0..15 (nearest the max first)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (t >= o) x += y;
    }
    const int before = x - tot;
    if (t < 16 && before < k_eff && k_eff <= x) {
      s_bin = t;
      s_above = before;
      s_binc = tot;
    }
  }
  __syncthreads();
  const uint32_t boct = (uint32_t)s_bin;
  int krem = k_eff - s_above;
  const bool whole = s_binc == krem;
  __syncthreads();
  // the threshold octave; octave 15 also holds everything further down
  uint32_t prefix = boct < 15u ? (top9 - boct) << 23 : 0u;
  uint32_t mask = boct < 15u ? 0xFF800000u : 0u;
  bool act[E];
#pragma unroll
  for (int e = 0; e < E; ++e) act[e] = boct < 15u ? oct[e] == boct : (oct[e] >= 15u && oct[e] < 16u);

  // 2. byte-wise radix passes inside the threshold octave
  if (!whole) {
    for (int hi = boct < 15u ? 22 : 31; hi >= 0; hi -= 8) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
      for (int i = lane; i < 256; i += 64) hist[wv][i] = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (act[e] && (key[e] & mask) == prefix) atomicAdd(&hist[wv][(key[e] >> lo) & dmask], 1);
      __syncthreads();
      if (t < 256) {
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += hist[w][t];
        s_tot[t] = tot;
      }
      __syncthreads();
      if (t < 64) {
        int h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = s_tot[4 * t + j];
        const int sl = h[0] + h[1] + h[2] + h[3];
        int x = sl;  // inclusive suffix sum over lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_down(x, o, kWave);
          if (t + o < 64) x += y;
        }
        int above = x - sl;
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
      prefix |= (uint32_t)b << lo;
      mask |= dmask << lo;
      __syncthreads();
      if (bc == krem) break;  // the whole threshold bin is taken
    }
  }

  // 3. keep octaves above the threshold one, keys above T, and the lowest-id ties
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t km = key[e] & mask;
    n_gt += oct[e] < boct || (act[e] && km > prefix);
    n_eq += act[e] && km == prefix;
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, s_wave, &tot);
  const int take_eq = max(0, min(n_eq, krem - eq_before));
  const int pos0 = block_exclusive_scan(n_gt + take_eq, s_wave, &tot);
  int pos = pos0, eq_taken = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t km = key[e] & mask;
    bool take = oct[e] < boct || (act[e] && km > prefix);
    if (act[e] && km == prefix) take = eq_taken++ < take_eq;
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
