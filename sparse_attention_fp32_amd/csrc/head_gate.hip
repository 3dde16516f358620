// a1: fp32 indexer head-gate  w[M,N] = hidden[M,K] @ W[K,N]   (N <= 16)
//
// The product of stkernel PR #227 ("indexer fp32 head-gate split-K"): at decode
// (M <= 16) a plain GEMM leaves almost every compute unit idle, so K is split
// into 128-row slices, one workgroup per slice.  Unlike the atomic float adds
// of that PR, the slice partials go to a workspace and the last workgroup to
// arrive (an integer ticket) adds them in slice order: deterministic, and the
// same bits for every row of a batch.  Above 16 rows each workgroup owns 16
// rows and walks all of K itself.
//
// HBM-bound work (2 FLOP per 4-byte hidden element), so this is plain fp32
// VALU arithmetic with LDS-staged tiles, not MFMA.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

constexpr int kSlice = 128;  // K rows per slice
constexpr int kRows = 16;    // output rows per workgroup
constexpr size_t kTicketBytes = 256;

// Thread t owns output (m = t / 16, n = t % 16) of the workgroup's 16 rows.
__global__ __launch_bounds__(256) void head_gate_kernel(const float* __restrict__ hidden,
                                                        const float* __restrict__ W,
                                                        float* __restrict__ w,
                                                        float* __restrict__ partial,
                                                        unsigned* __restrict__ ticket, int M,
                                                        int K, int N) {
  __shared__ float sh[kRows][kSlice + 1];
  __shared__ float sw[kSlice][16];
  __shared__ int s_last;
  const int t = threadIdx.x, m = t >> 4, n = t & 15;
  const int row0 = blockIdx.y * kRows;
  const int nsplit = gridDim.x;
  const int nslices = (K + kSlice - 1) / kSlice;
  float acc = 0.f;
  for (int sl = blockIdx.x; sl < nslices; sl += nsplit) {
    const int k0 = sl * kSlice;
    __syncthreads();
    for (int i = t; i < kRows * kSlice; i += 256) {
      const int mm = i / kSlice, kk = i % kSlice;
      const int gm = row0 + mm, gk = k0 + kk;
      sh[mm][kk] = (gm < M && gk < K) ? hidden[(size_t)gm * K + gk] : 0.f;
    }
    for (int i = t; i < kSlice * 16; i += 256) {
      const int kk = i >> 4, nn = i & 15;
      const int gk = k0 + kk;
      sw[kk][nn] = (gk < K && nn < N) ? W[(size_t)gk * N + nn] : 0.f;
    }
    __syncthreads();
#pragma unroll 16
    for (int kk = 0; kk < kSlice; ++kk) acc = fmaf(sh[m][kk], sw[kk][n], acc);
  }
  const int gm = row0 + m;
  if (nsplit == 1) {
    if (gm < M && n < N) w[(size_t)gm * N + n] = acc;
    return;
  }
  partial[blockIdx.x * 256 + t] = acc;
  __threadfence();  // release the partial before taking a ticket
  __syncthreads();
  if (t == 0) s_last = (atomicAdd(ticket, 1u) == (unsigned)(nsplit - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire every other workgroup's partial
  float tot = 0.f;
  for (int s = 0; s < nsplit; ++s) tot += partial[s * 256 + t];
  if (gm < M && n < N) w[(size_t)gm * N + n] = tot;
  if (t == 0) atomicExch(ticket, 0u);  // hand the workspace back zeroed
}

int split_count(int M, int K) {
  if (M > kRows) return 1;
  return (K + kSlice - 1) / kSlice;
}

}  // namespace

DSA_EXPORT size_t dsa_head_gate_workspace_size(int M, int K, int N) {
  (void)N;
  if (M <= 0 || K < 1) return 0;
  const int ns = split_count(M, K);
  if (ns <= 1) return 0;
  return kTicketBytes + (size_t)ns * 256 * sizeof(float);
}

DSA_EXPORT dsa_status dsa_head_gate(const float* hidden, const float* W, float* w, int M, int K,
                                    int N, void* ws, size_t ws_bytes, hipStream_t stream) {
  DSA_REQUIRE(N >= 1 && N <= DSA_MAX_INDEX_HEADS, DSA_ERR_INVALID_ARG,
              "dsa_head_gate: N=%d outside [1,%d]", N, DSA_MAX_INDEX_HEADS);
  DSA_REQUIRE(K >= 1, DSA_ERR_INVALID_ARG, "dsa_head_gate: K=%d < 1", K);
  DSA_REQUIRE(M >= 0, DSA_ERR_INVALID_ARG, "dsa_head_gate: M=%d < 0", M);
  if (M == 0) return DSA_OK;
  DSA_REQUIRE(hidden && W && w, DSA_ERR_INVALID_ARG, "dsa_head_gate: NULL tensor pointer");
  const size_t need = dsa_head_gate_workspace_size(M, K, N);
  DSA_REQUIRE(ws_bytes >= need && (need == 0 || ws), DSA_ERR_INVALID_ARG,
              "dsa_head_gate: workspace %zu bytes, need %zu", ws_bytes, need);
  const int ns = split_count(M, K);
  dim3 grid(ns, (M + kRows - 1) / kRows);
  unsigned* ticket = need ? (unsigned*)ws : nullptr;
  float* partial = need ? (float*)((char*)ws + kTicketBytes) : nullptr;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] head_gate M=%d K=%d N=%d grid=(%d,%d)\n", M, K, N, grid.x, grid.y);
  head_gate_kernel<<<grid, 256, 0, stream>>>(hidden, W, w, partial, ticket, M, K, N);
  return dsa::check_launch("dsa_head_gate");
}
