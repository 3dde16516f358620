// a1: fp32 indexer head-gate  w[M,N] = hidden[M,K] @ W[K,N]   (N <= 16)
//
// The product of stkernel PR #227 ("indexer fp32 head-gate split-K").  At
// decode (M <= 16) a plain GEMM leaves almost every compute unit idle and the
// PR splits K over programs that add their partials with float atomics.  Here
// each of the M rows (up to kRowMaxM of them) gets a 1024-thread workgroup
// that issues all of its loads at once (four 16-float rows of W and four hidden values per thread), keeps 16
// running sums per thread, and reduces them in a fixed order: a
// reduce-scatter over the wave (17 ALU-latency lane exchanges leave lane l with
// output j(l)),
// then the 16 waves' sums added in wave order.  Deterministic, and the same
// bits for a row whatever the batch.  Above kRowMaxM rows (prefill) each
// workgroup owns 16 rows: a [16,K] x [K,16] product on fp32 MFMA (v_mfma_f32_16x16x4_f32,
// fp32 products and sums) with the 16 waves splitting K and their 16x16
// partials added in wave order; K not a multiple of 16 takes a plain LDS-tiled
// loop.
//
// Either way the work is HBM-bound (2 FLOP per 4-byte element of hidden): at
// decode it is plain fp32 VALU arithmetic; at prefill the MFMA form only
// replaces 16 VALU FMAs per element with one quarter of an MFMA, so that the
// loop is nothing but loads in flight.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

constexpr int kSlice = 128;  // K rows per LDS tile (rows path)
constexpr int kRows = 16;    // output rows per workgroup (rows path)
constexpr int kRowThreads = 1024;
// Most rows taken one workgroup per row.  Each of those workgroups reads all
// of W (from L2), so the per-row form stops paying once the rows' W reads
// outweigh the 16-row MFMA form's single pass: measured per launch at K 4096,
// N 16, per-row against MFMA form, 6.1 vs 11.6 us at 17 rows, 6.4 vs 12.6 at
// 256, 10.3 vs 12.6 at 512, 17.4 vs 12.9 at 1024, 68 vs 15.8 at 4096.
constexpr int kRowMaxM = 512;
constexpr int kPerThread = 4;  // K elements per thread per pass (row path)

// One workgroup per output row m (M <= kRowMaxM).  Thread t takes k = t + 1024*i.
// N16: W rows are exactly 16 floats (four 16-byte loads per row).
template <bool N16>
__global__ __launch_bounds__(kRowThreads) void head_gate_row_kernel(const float* __restrict__ hidden,
                                                                    const float* __restrict__ W,
                                                                    float* __restrict__ w, int K,
                                                                    int N) {
  __shared__ float s_part[kRowThreads / 64][16];
  const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* hrow = hidden + (size_t)m * K;
  float acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = 0.f;
  for (int k0 = 0; k0 < K; k0 += kRowThreads * kPerThread) {
    float h[kPerThread];
    float4 wr[kPerThread][4];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int k = k0 + t + kRowThreads * i;
      const int kc = k < K ? k : K - 1;  // clamped: every load is in bounds
      h[i] = hrow[kc];
      if (N16) {
        const float4* wp = (const float4*)(W + (size_t)kc * 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) wr[i][c] = wp[c];
      } else {
        float tmp[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) tmp[n] = n < N ? W[(size_t)kc * N + n] : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          wr[i][c] = make_float4(tmp[4 * c], tmp[4 * c + 1], tmp[4 * c + 2], tmp[4 * c + 3]);
      }
      if (k >= K) h[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[4 * c + 0] = fmaf(h[i], wr[i][c].x, acc[4 * c + 0]);
        acc[4 * c + 1] = fmaf(h[i], wr[i][c].y, acc[4 * c + 1]);
        acc[4 * c + 2] = fmaf(h[i], wr[i][c].z, acc[4 * c + 2]);
        acc[4 * c + 3] = fmaf(h[i], wr[i][c].w, acc[4 * c + 3]);
      }
    }
  }
  // Reduce-scatter over the wave: each step keeps half of the running outputs
  // and adds the partner lane's copy of them (partners: l^32, l^16, then the
  // row mirror i <-> 15-i and half mirror i <-> 7-i, which also flip bits 3
  // and 2); lane l ends with output j(l) = 8*b5 + 4*b4 + 2*b3 + b2 summed over
  // 16 lanes, and the xor-2 and xor-1 steps finish the sum over all 64.
  float v8[8], v4[4], v2[2];
  {
    const bool hi = (lane >> 5) & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) v8[i] = (hi ? acc[8 + i] : acc[i]) + xor32(hi ? acc[i] : acc[8 + i]);
  }
  {
    const bool hi = (lane >> 4) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = (hi ? v8[4 + i] : v8[i]) + xor16(hi ? v8[i] : v8[4 + i]);
  }
  {
    const bool hi = (lane >> 3) & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v2[i] = (hi ? v4[2 + i] : v4[i]) + dpp_f<kDppMirror>(hi ? v4[i] : v4[2 + i]);
  }
  float v;
  {
    const bool hi = (lane >> 2) & 1;
    v = (hi ? v2[1] : v2[0]) + dpp_f<kDppHalfMirror>(hi ? v2[0] : v2[1]);
  }
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppXor1>(v);
  if ((lane & 3) == 0) {
    const int j = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 +
                  ((lane >> 2) & 1);
    s_part[wv][j] = v;
  }
  __syncthreads();
  if (t < N) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kRowThreads / 64; ++i) tot += s_part[i][t];
    w[(size_t)m * N + t] = tot;
  }
}

// 16 rows per workgroup, all of K through LDS tiles (M > kRowMaxM).  Thread t owns
// output (m = t / 16, n = t % 16).
__global__ __launch_bounds__(256) void head_gate_rows_kernel(const float* __restrict__ hidden,
                                                             const float* __restrict__ W,
                                                             float* __restrict__ w, int M, int K,
                                                             int N) {
  __shared__ float sh[kRows][kSlice + 1];
  __shared__ float sw[kSlice][16];
  const int t = threadIdx.x, m = t >> 4, n = t & 15;
  const int row0 = blockIdx.x * kRows;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += kSlice) {
    __syncthreads();
    for (int i = t; i < kRows * kSlice; i += 256) {
      const int mm = i / kSlice, kk = i % kSlice;
      const int gm = row0 + mm, gk = k0 + kk;
      const float v = hidden[(size_t)(gm < M ? gm : M - 1) * K + (gk < K ? gk : K - 1)];
      sh[mm][kk] = (gm < M && gk < K) ? v : 0.f;
    }
    for (int i = t; i < kSlice * 16; i += 256) {
      const int kk = i >> 4, nn = i & 15;
      const int gk = k0 + kk;
      const float v = W[(size_t)(gk < K ? gk : K - 1) * N + (nn < N ? nn : N - 1)];
      sw[kk][nn] = (gk < K && nn < N) ? v : 0.f;
    }
    __syncthreads();
#pragma unroll 16
    for (int kk = 0; kk < kSlice; ++kk) acc = fmaf(sh[m][kk], sw[kk][n], acc);
  }
  const int gm = row0 + m;
  if (gm < M && n < N) w[(size_t)gm * N + n] = acc;
}

typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 16;  // waves over K per workgroup (MFMA path)

// 16 rows per workgroup (M > kRowMaxM, K % 16 == 0).  MFMA 16x16x4 f32: lane l holds
// A[l % 16][l / 16] = hidden[m0 + l % 16][k], B[l / 16][l % 16] = W[k][l % 16],
// and D[4 (l / 16) + r][l % 16] in acc[r].  A float4 of a hidden row feeds four
// MFMAs: for c < 4 the K index of lane group j is k0 + 4 j + c.  Wave wv takes
// the 16-wide K steps [s0, s1) in passes of U steps, two register sets in
// turn: the loads of the next pass are issued before the MFMAs of the current
// one, so the MFMAs run while the next rows stream in.  The MFMAs still take
// the steps in ascending order.
template <int U>  // K steps per pass
__global__ __launch_bounds__(kGateWaves * 64) void head_gate_mfma_kernel(
    const float* __restrict__ hidden, const float* __restrict__ W, float* __restrict__ w, int M,
    int K, int N) {
  __shared__ f32x4_v s_red[kGateWaves][64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int i = lane & 15, j = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const float* hrow = hidden + (size_t)min(m0 + i, M - 1) * K;
  const int nsteps = K / 16;
  const int s0 = nsteps * wv / kGateWaves, s1 = nsteps * (wv + 1) / kGateWaves;
  const int ncol = i < N ? i : N - 1;
  const float bmask = i < N ? 1.f : 0.f;
  f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
  // (steps past s1 are loaded, clamped to s1 - 1, and not used)
  auto load = [&](float4 (&h)[U], float (&b)[U][4], int sb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = min(sb + u, s1 - 1) * 16;
      h[u] = *(const float4*)(hrow + k0 + 4 * j);
#pragma unroll
      for (int c = 0; c < 4; ++c) b[u][c] = W[(size_t)(k0 + 4 * j + c) * N + ncol];
    }
  };
  auto mma = [&](const float4 (&h)[U], const float (&b)[U][4], int sb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (sb + u < s1) {
        const float hv[4] = {h[u].x, h[u].y, h[u].z, h[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(hv[c], b[u][c] * bmask, acc, 0, 0, 0);
      }
    }
  };
  float4 ha[U], hb[U];
  float ba[U][4], bb[U][4];
  if (s0 < s1) load(ha, ba, s0);
  for (int sb = s0; sb < s1; sb += 2 * U) {
    if (sb + U < s1) load(hb, bb, sb + U);
    mma(ha, ba, sb);
    if (sb + U >= s1) break;
    if (sb + 2 * U < s1) load(ha, ba, sb + 2 * U);
    mma(hb, bb, sb + U);
  }
  s_red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    f32x4_v v = s_red[0][lane];
#pragma unroll
    for (int x = 1; x < kGateWaves; ++x) v += s_red[x][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 4 * j + r;
      if (m < M && i < N) w[(size_t)m * N + i] = v[r];
    }
  }
}

}  // namespace

DSA_EXPORT size_t dsa_head_gate_workspace_size(int M, int K, int N) {
  (void)M;
  (void)K;
  (void)N;
  return 0;
}

DSA_EXPORT dsa_status dsa_head_gate(const float* hidden, const float* W, float* w, int M, int K,
                                    int N, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  DSA_REQUIRE(N >= 1 && N <= DSA_MAX_INDEX_HEADS, DSA_ERR_INVALID_ARG,
              "dsa_head_gate: N=%d outside [1,%d]", N, DSA_MAX_INDEX_HEADS);
  DSA_REQUIRE(K >= 1, DSA_ERR_INVALID_ARG, "dsa_head_gate: K=%d < 1", K);
  DSA_REQUIRE(M >= 0, DSA_ERR_INVALID_ARG, "dsa_head_gate: M=%d < 0", M);
  if (M == 0) return DSA_OK;
  DSA_REQUIRE(hidden && W && w, DSA_ERR_INVALID_ARG, "dsa_head_gate: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_head_gate", hidden, W, w, ws);
  if (dsa::trace_enabled()) fprintf(stderr, "[dsa] head_gate M=%d K=%d N=%d\n", M, K, N);
  if (dsa::dry_run()) return DSA_OK;
  if (M <= kRowMaxM)
    if (N == 16)
      head_gate_row_kernel<true><<<M, kRowThreads, 0, stream>>>(hidden, W, w, K, N);
    else
      head_gate_row_kernel<false><<<M, kRowThreads, 0, stream>>>(hidden, W, w, K, N);
  else if (K % 16 == 0)
    head_gate_mfma_kernel<4><<<(M + kRows - 1) / kRows, kGateWaves * 64, 0, stream>>>(hidden, W, w,
                                                                                   M, K, N);
  else
    head_gate_rows_kernel<<<(M + kRows - 1) / kRows, 256, 0, stream>>>(hidden, W, w, M, K, N);
  return dsa::check_launch("dsa_head_gate");
}
