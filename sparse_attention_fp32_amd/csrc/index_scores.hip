// a3: index scores  s[q,p] = sum_h w[q,h] * relu(<qi[q,h,:], key[p,:]>)  plus
// candidate validity (Atlas glm5next_dsa page, "Shape of the pipeline").
//
// Per query this is a [H x D] x [D x P] contraction (16 heads x 128 dims against
// every pooled key of the request), 16 FLOP per key byte -- on the fp32 VALU
// ridge, so it runs on MFMA: v_mfma_f32_16x16x32_bf16 with the heads as M and
// 16 pools as N.  The query's A operand stays in registers; each lane streams
// its pools' key rows straight from HBM into the B-operand layout (16 bytes per
// lane per k-step, a 64-byte run of one key row per lane group), four 16-pool
// tiles per wave in flight.  The relu, head weighting and head sum happen on
// the accumulator: each lane holds 4 heads of one pool; two permlane swaps finish
// the sum in a fixed order.
//
// Gated variant (dsa_index_scores_gated, fused decode path): the head weights
// arrive as split-K partials of the head-gate (one per 128-wide K slice); each
// workgroup adds them in slice order while its key rows load, and the first
// workgroup of each query stores the sum as w.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

constexpr int kTiles = 4;                  // 16-pool tiles per wave
constexpr int kPoolsPerWG = 4 * kTiles * 16;  // 4 waves (= 256, one slot per thread)
static_assert(kPoolsPerWG == 256, "the sentinel-only path gives each thread one slot");

constexpr int kMaxGateSlices = 64;  // 16 slice groups x 4 per thread

template <int KS, bool GATED>  // D / 32 k-steps; w given as head-gate partials
__global__ __launch_bounds__(256) void index_scores_kernel(
    const uint16_t* __restrict__ qi, const float* __restrict__ w,
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ pool_start,
    const uint8_t* __restrict__ pool_valid, const int32_t* __restrict__ pool_off,
    const int32_t* __restrict__ n_pools, const int32_t* __restrict__ q_req,
    const int32_t* __restrict__ q_pos, int H, int kpool, int pstride, float* __restrict__ scores,
    uint8_t* __restrict__ cand, int nslices, float* __restrict__ w_out) {
  constexpr int D = KS * 32;
  const int q = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // Head-gate partials first (gated variant): the oldest loads, so the
  // reduction below waits for them alone while the key rows stream in.
  float gp[4];
  if (GATED) {
    const int Q = gridDim.y;
    const int h = threadIdx.x & 15, g = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = min(g + 16 * i, nslices - 1);
      gp[i] = w[((int64_t)sl * Q + q) * H + min(h, H - 1)];
    }
  }
  const int r = q_req[q];
  const int P = n_pools[r];
  const int64_t base = pool_off[r];
  const int qp = q_pos[q];
  const int wg0 = blockIdx.x * kPoolsPerWG;
  const int tile0 = wg0 + wave * (kTiles * 16);
  // A workgroup past the request's last pool (ragged batches: the row is as
  // long as the longest request's) writes its slots' sentinels and leaves,
  // unless it is the one that stores w.
  if (wg0 >= P && !(GATED && w_out && blockIdx.x == 0)) {
    const int p = wg0 + (int)threadIdx.x;  // kPoolsPerWG == blockDim.x
    if (p < pstride) {
      scores[(int64_t)q * pstride + p] = -INFINITY;
      cand[(int64_t)q * pstride + p] = 0;
    }
    return;
  }

  // Key rows: the long-latency HBM stream.  Every load is issued, unconditional
  // and together: pool indices are clamped to the request's last pool (a
  // request without pools reads this query's qi row instead), and pools past
  // the end are masked below.
  const uint16_t* kb = P > 0 ? keys + base * D : qi + (int64_t)q * H * D;
  const int32_t* sb = P > 0 ? pool_start + base : q_pos;
  const uint8_t* vb = P > 0 ? pool_valid + base : (const uint8_t*)q_pos;
  const int plast = max(P - 1, 0);
  uint4 b[kTiles][KS];
  int ps[kTiles], pv[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const int p = min(tile0 + tt * 16 + col, plast);
    const uint16_t* krow = kb + (int64_t)p * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) b[tt][kk] = *(const uint4*)(krow + kk * 32);
    ps[tt] = sb[p];
    pv[tt] = vb[p];
  }
  // A operand: row m = head col, k = kk*32 + grp*8 + j.  Rows past H repeat
  // head H-1; their weight is zero below.
  bf16x8_t a[KS];
  const uint16_t* qrow = qi + ((int64_t)q * H + min(col, H - 1)) * D + grp * 8;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) a[kk] = as_bf16x8(*(const uint4*)(qrow + kk * 32));
  float wr[4];
  if (GATED) {
    // w[q, h] = sum over slices of part[sl][q][h]: thread (group g, head h)
    // adds slices g, g+16, g+32, g+48; the 16 group sums go in group order.
    __shared__ float s_red[16][16];
    __shared__ float s_w[16];
    const int t = threadIdx.x, h = t & 15, g = t >> 4;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += g + 16 * i < nslices ? gp[i] : 0.f;
    s_red[g][h] = acc;
    __syncthreads();
    if (t < 16) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += s_red[j][t];
      s_w[t] = sum;
      if (w_out && blockIdx.x == 0 && t < H) w_out[(int64_t)q * H + t] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = grp * 4 + i < H ? s_w[grp * 4 + i] : 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = grp * 4 + i;
      const float v = w[(int64_t)q * H + (h < H ? h : H - 1)];
      wr[i] = h < H ? v : 0.f;
    }
  }

#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) acc = mfma16x16x32(a[kk], as_bf16x8(b[tt][kk]), acc);
    // acc[i] = <qi[head grp*4+i], key[pool col]>
    float s = fmaxf(acc[0], 0.f) * wr[0];
    s += fmaxf(acc[1], 0.f) * wr[1];
    s += fmaxf(acc[2], 0.f) * wr[2];
    s += fmaxf(acc[3], 0.f) * wr[3];
    s = rows_sum(s);  // the four lane rows hold four heads each
    if (s == 0.f) s = 0.f;  // store -0 as +0
    const int p = tile0 + tt * 16 + col;
    const bool c = p < P && pv[tt] != 0 && ps[tt] + kpool - 1 <= qp;
    if (p < pstride) {
      if (grp == 0) scores[(int64_t)q * pstride + p] = c ? s : -INFINITY;
      if (grp == 1) cand[(int64_t)q * pstride + p] = (uint8_t)c;
    }
  }
}

}  // namespace

namespace {

dsa_status launch_scores(const uint16_t* qi, const float* w, int nslices, float* w_out,
                         const uint16_t* keys, const int32_t* pool_start,
                         const uint8_t* pool_valid, const int32_t* pool_off,
                         const int32_t* n_pools, const int32_t* q_req, const int32_t* q_pos,
                         int Q, int H, int D, int kpool, int pstride, float* scores,
                         uint8_t* cand, hipStream_t stream, const char* who) {
  DSA_REQUIRE(H >= 1 && H <= DSA_MAX_INDEX_HEADS, DSA_ERR_INVALID_ARG, "%s: H=%d outside [1,%d]",
              who, H, DSA_MAX_INDEX_HEADS);
  DSA_REQUIRE(kpool >= 1 && kpool <= DSA_MAX_KPOOL, DSA_ERR_INVALID_ARG,
              "%s: kpool=%d outside [1,%d]", who, kpool, DSA_MAX_KPOOL);
  DSA_REQUIRE(D == 32 || D == 64 || D == 128 || D == 256, DSA_ERR_UNSUPPORTED,
              "%s: D=%d not in {32,64,128,256}", who, D);
  DSA_REQUIRE(pstride >= 1, DSA_ERR_INVALID_ARG, "%s: pstride=%d < 1", who, pstride);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "%s: Q=%d < 0", who, Q);
  DSA_REQUIRE(nslices >= 0 && nslices <= kMaxGateSlices, DSA_ERR_INVALID_ARG,
              "%s: %d head-gate slices outside [1,%d]", who, nslices, kMaxGateSlices);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(qi && w && keys && pool_start && pool_valid && pool_off && n_pools && q_req &&
                  q_pos && scores && cand,
              DSA_ERR_INVALID_ARG, "%s: NULL tensor pointer", who);
  DSA_REQUIRE_ALIGNED(who, qi, w, w_out, keys, pool_start, pool_valid, pool_off, n_pools, q_req,
                      q_pos, scores, cand);
  dim3 grid((pstride + kPoolsPerWG - 1) / kPoolsPerWG, Q);
  DSA_REQUIRE(grid.y <= 65535u, DSA_ERR_UNSUPPORTED, "%s: Q=%d above 65535", who, Q);
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] %s Q=%d H=%d D=%d pstride=%d slices=%d grid=(%d,%d)\n", who, Q, H, D,
            pstride, nslices, grid.x, grid.y);
#define DSA_LAUNCH_IS(KS, G)                                                               \
  index_scores_kernel<KS, G><<<grid, 256, 0, stream>>>(qi, w, keys, pool_start, pool_valid, \
                                                       pool_off, n_pools, q_req, q_pos, H,  \
                                                       kpool, pstride, scores, cand, nslices, w_out)
#define DSA_LAUNCH_IS_D(G)             \
  switch (D / 32) {                    \
    case 1: DSA_LAUNCH_IS(1, G); break; \
    case 2: DSA_LAUNCH_IS(2, G); break; \
    case 4: DSA_LAUNCH_IS(4, G); break; \
    default: DSA_LAUNCH_IS(8, G); break; \
  }
  if (nslices > 0) {
    DSA_LAUNCH_IS_D(true);
  } else {
    DSA_LAUNCH_IS_D(false);
  }
#undef DSA_LAUNCH_IS_D
#undef DSA_LAUNCH_IS
  return dsa::check_launch(who);
}

}  // namespace

DSA_EXPORT dsa_status dsa_index_scores(const uint16_t* qi, const float* w, const uint16_t* keys,
                                       const int32_t* pool_start, const uint8_t* pool_valid,
                                       const int32_t* pool_off, const int32_t* n_pools,
                                       const int32_t* q_req, const int32_t* q_pos, int Q, int H,
                                       int D, int kpool, int pstride, float* scores,
                                       uint8_t* cand, hipStream_t stream) {
  return launch_scores(qi, w, 0, nullptr, keys, pool_start, pool_valid, pool_off, n_pools, q_req,
                       q_pos, Q, H, D, kpool, pstride, scores, cand, stream, "dsa_index_scores");
}

DSA_EXPORT dsa_status dsa_index_scores_gated(const uint16_t* qi, const float* gate_part,
                                             int nslices, float* w, const uint16_t* keys,
                                             const int32_t* pool_start,
                                             const uint8_t* pool_valid, const int32_t* pool_off,
                                             const int32_t* n_pools, const int32_t* q_req,
                                             const int32_t* q_pos, int Q, int H, int D,
                                             int kpool, int pstride, float* scores,
                                             uint8_t* cand, hipStream_t stream) {
  DSA_REQUIRE(nslices >= 1, DSA_ERR_INVALID_ARG, "dsa_index_scores_gated: nslices=%d < 1",
              nslices);
  return launch_scores(qi, gate_part, nslices, w, keys, pool_start, pool_valid, pool_off, n_pools,
                       q_req, q_pos, Q, H, D, kpool, pstride, scores, cand, stream,
                       "dsa_index_scores_gated");
}
