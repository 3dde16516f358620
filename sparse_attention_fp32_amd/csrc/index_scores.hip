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
//
// Prefill-sized batches (many queries of one sequence scanning the same keys)
// take the query-block form below: the keys of a 256-pool block stay in
// registers while the workgroup walks 8 consecutive queries, so the call is a
// dense [Q*H x D] x [D x P] contraction instead of Q separate key streams.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

constexpr int kTiles = 4;                  // 16-pool tiles per wave
constexpr int kPoolsPerWG = 4 * kTiles * 16;  // 4 waves (= 256, one slot per thread)
static_assert(kPoolsPerWG == 256, "the sentinel-only path gives each thread one slot");
static_assert(kTiles == 4, "the score stores give each lane group one tile");

constexpr int kMaxGateSlices = 64;  // 16 slice groups x 4 per thread
constexpr int kQB = 8;              // queries per workgroup in the query-block form
static_assert(kQB <= 16 && 16 % kQB == 0, "the weight table has 16 rows of 16 threads");
// The query-block form is chosen for batches of many queries (prefill-sized)
// when its grid still gives every compute unit a workgroup.
constexpr int kQBlockMinQ = 256;
constexpr long long kQBlockMinWG = 256;

__device__ __forceinline__ uint64_t ballot_any(bool p) { return __builtin_amdgcn_ballot_w64(p); }

typedef __attribute__((address_space(3))) void lds_void_t;

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
    const int h = threadIdx.x & 15, g = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = min(g + 16 * i, nslices - 1);
      gp[i] = w[((int64_t)q * nslices + sl) * H + min(h, H - 1)];
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

  // after the head sum every lane of column col holds tile tt's score for
  // pool tile0 + 16tt + col; lane (col, grp) keeps tile grp's, so each wave
  // stores its 64 pools with one score and one flag instruction
  float so = -INFINITY;
  bool co = false;
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
    if (grp == tt) {
      so = c ? s : -INFINITY;
      co = c;
    }
  }
  const int p = tile0 + lane;
  if (p < pstride) {
    scores[(int64_t)q * pstride + p] = so;
    cand[(int64_t)q * pstride + p] = (uint8_t)co;
  }
}

// Query-block form: workgroup (256-pool block, block of kQB consecutive
// queries).  When the block's queries share one request (prefill: many
// queries of one sequence) the key rows, their starts and validity load once
// and stay in registers while the workgroup walks its queries, so the pooled
// keys are read once per query block instead of once per query and the
// contraction [kQB*H x D] x [D x 256] runs from registers.  A block whose
// queries span requests reloads the keys whenever the request changes (the
// result is the same, only slower).  Per (query, pool) the arithmetic is the
// per-query kernel's, in the same order: the same MFMA chain over k, the same
// relu / weight / head sum, and the gate partials added in the same grouping,
// so both forms give the same bits.  A wave whose 64 pools hold no candidate
// for the query (every pool past the request's end, invalid, or after the
// query's position) skips its MFMAs.
template <int KS, bool GATED, int NS>  // NS: most head-gate slices (1, 16, 32 or 64)
__global__ __launch_bounds__(256) void index_scores_qblock_kernel(
    const uint16_t* __restrict__ qi, const float* __restrict__ w,
    const uint16_t* __restrict__ keys, const int32_t* __restrict__ pool_start,
    const uint8_t* __restrict__ pool_valid, const int32_t* __restrict__ pool_off,
    const int32_t* __restrict__ n_pools, const int32_t* __restrict__ q_req,
    const int32_t* __restrict__ q_pos, int Q, int H, int kpool, int pstride,
    float* __restrict__ scores, uint8_t* __restrict__ cand, int nslices,
    float* __restrict__ w_out) {
  constexpr int D = KS * 32;
  constexpr int kRowChunks = D / 8;  // 16-byte chunks of one head's qi row
  __shared__ float s_w[kQB][16];     // head weights of the block's queries
  // the block's qi rows [query][head (16 slots)][chunk], chunk k of head h
  // stored at k ^ (h mod kRowChunks) so that the 16 heads of one A-operand
  // read fall in distinct banks
  __shared__ uint4 s_qi[kQB * 16 * kRowChunks];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // Workgroup -> (pool block, query block), XCD-aware: workgroups go to the
  // eight XCDs in turn, so the pool blocks of one query block are given ids
  // eight apart -- the same XCD, dispatched together -- and its qi rows are
  // fetched into that XCD's L2 once.  The grid's query blocks are padded to
  // a multiple of 8; the padding workgroups leave at once.
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int pblk = (lin >> 3) % gridDim.x;
  const int qblk = ((lin >> 3) / gridDim.x) * 8 + (lin & 7);
  const int qb0 = qblk * kQB;
  if (qb0 >= Q) return;
  const int nq = min(kQB, Q - qb0);
  const int wg0 = pblk * kPoolsPerWG;
  const int tile0 = wg0 + wave * (kTiles * 16);
  // thread (query j, head h) of the weight table
  // (with fewer than 16 queries per block the upper threads repeat the lower)
  const int wj = (t >> 4) % kQB, wh = t & 15;
  const bool wown = (t >> 4) < kQB;  // this thread's entry is the one kept
  const int wq = qb0 + min(wj, nq - 1);
  // weights first (the oldest loads): head-gate partials of slices g, g+16,
  // g+32, g+48 for every slice group g, or w itself
  float gp[GATED ? NS : 1];
  if (GATED) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      gp[sl] = w[((int64_t)wq * nslices + min(sl, nslices - 1)) * H + min(wh, H - 1)];
  } else {
    gp[0] = w[(int64_t)wq * H + min(wh, H - 1)];
  }
  // the block's qi rows straight into LDS (no registers held): instruction i
  // of wave v fills the 64 chunks from (4i + v) * 64 on; rows past the block
  // or past H repeat the last query or head
  for (int c0 = wave * 64; c0 < kQB * 16 * kRowChunks; c0 += 4 * 64) {
    const int c = c0 + lane;
    const int j = c / (16 * kRowChunks), h = (c / kRowChunks) % 16;
    const int k = (c % kRowChunks) ^ (h % kRowChunks);
    const uint16_t* src =
        qi + ((int64_t)(qb0 + min(j, nq - 1)) * H + min(h, H - 1)) * D + k * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(s_qi + c0), 16, 0, 0);
  }
  // the block's queries: lane j (mod 16) holds query qb0 + j's request and position
  const int gq = qb0 + min(col, nq - 1);
  const int greq = q_req[gq], gpos = q_pos[gq];
  const int r0 = __builtin_amdgcn_readfirstlane(greq);
  const bool uniform = ballot_any(greq != r0) == 0;

  // key rows of request r: every load unconditional, pool indices clamped to
  // the request's last pool (a request without pools reads the first query's
  // qi row instead; its pools are masked below)
  uint4 b[kTiles][KS] = {};
  int ps[kTiles] = {}, pv[kTiles] = {};
  int P = 0;
  // per tile: the pool exists and is valid, and the last position it needs
  bool pok[kTiles];
  int plim[kTiles];
  // Take delivery of the key rows (one wait) and derive the pools' limits.
  // On this chip stores count in the same counter as loads, so no register
  // of a load may still be pending inside the query loop: a wait for it
  // would also wait for the stores of the queries before.
  auto deliver_keys = [&]() {
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        asm volatile("" ::"v"(b[tt][kk].x), "v"(b[tt][kk].y), "v"(b[tt][kk].z), "v"(b[tt][kk].w));
      pok[tt] = tile0 + tt * 16 + col < P && pv[tt] != 0;
      plim[tt] = ps[tt] + kpool - 1;
    }
  };
  auto load_keys = [&](int r) {
    P = n_pools[r];
    const int64_t base = pool_off[r];
    const uint16_t* kb = P > 0 ? keys + base * D : qi + (int64_t)qb0 * H * D;
    const int32_t* sb = P > 0 ? pool_start + base : q_pos;
    const uint8_t* vb = P > 0 ? pool_valid + base : (const uint8_t*)q_pos;
    const int plast = max(P - 1, 0);
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      const int p = min(tile0 + tt * 16 + col, plast);
      const uint16_t* krow = kb + (int64_t)p * D + grp * 8;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) b[tt][kk] = *(const uint4*)(krow + kk * 32);
      ps[tt] = sb[p];
      pv[tt] = vb[p];
    }
  };
  int rcur = -1;
  if (uniform) {
    load_keys(r0);
    rcur = r0;
    // nothing of this block's pools exists for the request: sentinels only
    // (unless this workgroup stores w)
    if (wg0 >= P && !(GATED && w_out && pblk == 0)) {
      const int p = wg0 + t;  // kPoolsPerWG == blockDim.x
      if (p < pstride)
        for (int j = 0; j < nq; ++j) {
          scores[(int64_t)(qb0 + j) * pstride + p] = -INFINITY;
          cand[(int64_t)(qb0 + j) * pstride + p] = 0;
        }
      // the qi rows' DMA into LDS lands before the workgroup gives its LDS up
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
  }
  // weight table: the same grouping as the per-query kernel (per slice
  // group g the slices g, g+16, g+32, g+48 in order, then the 16 group sums
  // in group order)
  {
    float sum;
    if (GATED) {
      sum = 0.f;
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (g + 16 * i < NS) acc += g + 16 * i < nslices ? gp[g + 16 * i] : 0.f;
        sum += acc;
      }
      if (w_out && pblk == 0 && wown && wj < nq && wh < H)
        w_out[(int64_t)(qb0 + wj) * H + wh] = sum;
    } else {
      sum = gp[0];
    }
    if (wown) s_w[wj][wh] = wh < H ? sum : 0.f;
  }
  // (unconditional: the compiler's wait tracking does not follow the uniform
  // branch, so a delivery inside it would leave the keys pending in the loop;
  // a block that spans requests has loaded nothing yet and reloads below)
  deliver_keys();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the qi rows are in LDS
  __syncthreads();
  const int ha = min(col, H - 1);  // A-operand row of this lane (rows past H repeat H-1)

  for (int j = 0; j < nq; ++j) {
    const int q = qb0 + j;
    const int r = __builtin_amdgcn_readlane(greq, j);
    const int qp = __builtin_amdgcn_readlane(gpos, j);
    if (r != rcur) {  // a block that spans requests (uniform over the workgroup)
      load_keys(r);
      deliver_keys();
      rcur = r;
    }
    float wr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = s_w[j][grp * 4 + i];
    // A operand: row m = head col, k = kk*32 + grp*8 + e
    bf16x8_t a[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      a[kk] = as_bf16x8(
          s_qi[(j * 16 + ha) * kRowChunks + ((kk * 4 + grp) ^ (ha % kRowChunks))]);
    // after the head sum every lane of column col holds tile tt's score for
    // pool tile0 + 16tt + col; lane (col, grp) keeps tile grp's, so each
    // wave stores its 64 pools with one score and one flag instruction
    bool c[kTiles];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      c[tt] = pok[tt] && plim[tt] <= qp;
      any |= c[tt];
    }
    float sv[kTiles] = {0.f, 0.f, 0.f, 0.f};
    if (ballot_any(any) != 0) {  // the four tiles' chains interleave
      f32x4_t acc[kTiles];
#pragma unroll
      for (int tt = 0; tt < kTiles; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt)
          acc[tt] = mfma16x16x32(a[kk], as_bf16x8(b[tt][kk]), acc[tt]);
#pragma unroll
      for (int tt = 0; tt < kTiles; ++tt) {
        float s = fmaxf(acc[tt][0], 0.f) * wr[0];
        s += fmaxf(acc[tt][1], 0.f) * wr[1];
        s += fmaxf(acc[tt][2], 0.f) * wr[2];
        s += fmaxf(acc[tt][3], 0.f) * wr[3];
        s = rows_sum(s);
        if (s == 0.f) s = 0.f;  // store -0 as +0
        sv[tt] = s;
      }
    }
    float so = -INFINITY;
    bool co = false;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt)
      if (grp == tt) {
        so = c[tt] ? sv[tt] : -INFINITY;
        co = c[tt];
      }
    const int p = tile0 + lane;
    if (p < pstride) {
      scores[(int64_t)q * pstride + p] = so;
      cand[(int64_t)q * pstride + p] = (uint8_t)co;
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
  DSA_REQUIRE(Q <= 65535, DSA_ERR_UNSUPPORTED, "%s: Q=%d above 65535", who, Q);
  // many queries (prefill): the query-block form, whenever its grid still
  // fills the chip
  const int pblocks = (pstride + kPoolsPerWG - 1) / kPoolsPerWG;
  const int qblocks = (Q + kQB - 1) / kQB;
  const bool qblock = Q >= kQBlockMinQ && (long long)pblocks * qblocks >= kQBlockMinWG;
  // (query blocks padded to a multiple of 8 for the XCD-aware order)
  const dim3 grid(pblocks, qblock ? (qblocks + 7) / 8 * 8 : Q);
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] %s Q=%d H=%d D=%d pstride=%d slices=%d grid=(%d,%d)%s\n", who, Q, H, D,
            pstride, nslices, grid.x, grid.y, qblock ? " query-block" : "");
#define DSA_LAUNCH_QB(KS, G, NS)                                                         \
  index_scores_qblock_kernel<KS, G, NS><<<grid, 256, 0, stream>>>(                         \
      qi, w, keys, pool_start, pool_valid, pool_off, n_pools, q_req, q_pos, Q, H, kpool,   \
      pstride, scores, cand, nslices, w_out)
#define DSA_LAUNCH_QB_NS(KS)            \
  if (nslices == 0)                     \
    DSA_LAUNCH_QB(KS, false, 1);        \
  else if (nslices == 1)                \
    DSA_LAUNCH_QB(KS, true, 1);         \
  else if (nslices <= 16)               \
    DSA_LAUNCH_QB(KS, true, 16);        \
  else if (nslices <= 32)               \
    DSA_LAUNCH_QB(KS, true, 32);        \
  else                                  \
    DSA_LAUNCH_QB(KS, true, 64)
#define DSA_LAUNCH_IS(KS)                                                                      \
  if (nslices > 0)                                                                             \
    index_scores_kernel<KS, true><<<grid, 256, 0, stream>>>(                                   \
        qi, w, keys, pool_start, pool_valid, pool_off, n_pools, q_req, q_pos, H, kpool,        \
        pstride, scores, cand, nslices, w_out);                                                \
  else                                                                                         \
    index_scores_kernel<KS, false><<<grid, 256, 0, stream>>>(                                  \
        qi, w, keys, pool_start, pool_valid, pool_off, n_pools, q_req, q_pos, H, kpool,        \
        pstride, scores, cand, nslices, w_out)
#define DSA_SWITCH_D(LAUNCH)        \
  switch (D / 32) {                 \
    case 1: LAUNCH(1); break;       \
    case 2: LAUNCH(2); break;       \
    case 4: LAUNCH(4); break;       \
    default: LAUNCH(8); break;      \
  }
  if (dsa::dry_run()) return DSA_OK;
  if (qblock) {
    DSA_SWITCH_D(DSA_LAUNCH_QB_NS)
  } else {
    DSA_SWITCH_D(DSA_LAUNCH_IS)
  }
#undef DSA_SWITCH_D
#undef DSA_LAUNCH_IS
#undef DSA_LAUNCH_QB_NS
#undef DSA_LAUNCH_QB
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
