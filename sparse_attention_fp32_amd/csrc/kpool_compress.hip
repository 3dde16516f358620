// a2: gated pool compression + k_norm (bias-bearing LayerNorm), fused.
//
// Atlas glm5next_dsa page, "Traps carried from Slice 8": the pool softmax runs
// over the pool-slot axis separately per channel; pooling starts at the first
// valid row; a pool counts only if all kpool slots are valid (a trailing
// partial pool is no pool); k_norm is an nn.LayerNorm with a bias.  The page
// runs compression and an in-place bf16 LayerNorm as two kernels; here the
// LayerNorm is applied to the fp32 pooled row in registers and the key is
// rounded to bf16 once.
//
// Layout: one pool is handled by D/8 lanes, each owning 8 channels (one 16-byte
// load per slot row), so a wave streams 64/(D/8) pools at once with fully
// coalesced row reads.  Per-channel slot softmax is lane-local; the LayerNorm
// mean and variance are DPP reductions over the pool's lanes.
// HBM-bound (2*kpool*D*2 bytes in, D*2 out per pool): no MFMA.
//
// Incremental mode (a decode step that appended rows) walks the rewritten
// pools from the last one down and needs two dependent loads per request:
// the request's geometry, then the first valid row together with the rows of
// the pool ending at the newest row (which is where a step's work lies when
// its newest row completes a pool).  The first valid row comes from slot 0 of
// the earlier call whenever that slot holds a pool starting before new_from.
//
// Live lengths: with seq_len, request r holds seq_len[r] rows of its region
// (the rest of the region is not read).  Without ln_w / ln_b the rows were
// normalised when stored (per-token k_normed) and the pooled row is rounded to
// bf16 with no LayerNorm.
//
// Fused decode variant (dsa_gate_compress): the head-gate of the same step is
// independent of the compression, so the same launch also runs it, split over
// K (stkernel PR #227's split-K) in workgroups placed after the compression
// ones.  Each writes the partial products of one 128-wide K slice for 16 rows;
// the index-score kernel adds the slices in a fixed order, so the gate leaves
// the launch chain and stays deterministic.
#include <limits.h>

#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

// First valid row of a request (request-local), or -1.
//
// The request's bytes valid[row0, row0 + T) are read as the 16-byte chunks of
// the array that hold them (the array starts 16-byte aligned).  Bytes of a
// chunk outside the request are masked off; the chunk holding the request's
// last byte is read byte by byte with clamped addresses, and lanes past it
// read kScanPad, so no access passes the request's end (the array may end
// there).  Rounds of 256 * U chunks, all loads of a round in flight: a first
// round of 4 KiB (a request that starts valid is found at once), then 16 KiB
// rounds (wider rounds cost the kernel a wave of occupancy at kpool 4), so
// left padding of 64 Ki rows costs five round trips rather than sixteen.
__device__ uint4 kScanPad;
__device__ __forceinline__ uint64_t nz_bytes(uint32_t lo, uint32_t hi) {
  // bit 8i+7 set for each nonzero byte i of the 8 bytes lo | hi << 32
  const uint32_t a = (((lo & 0x7f7f7f7fu) + 0x7f7f7f7fu) | lo) & 0x80808080u;
  const uint32_t b = (((hi & 0x7f7f7f7fu) + 0x7f7f7f7fu) | hi) & 0x80808080u;
  return a | (uint64_t)b << 32;
}
__device__ __forceinline__ uint64_t bytes_below(int n) {  // bytes [0, n) of 8
  return n <= 0 ? 0ull : n >= 8 ? ~0ull : (1ull << (8 * n)) - 1;
}

template <int U>
__device__ int scan_round(const uint4* __restrict__ vc, int64_t jb, int64_t j1,
                          uint4 last, int64_t row0, int64_t end) {
  const int t = threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = jb + u * 256 + t;
    v[u] = *(j < j1 ? vc + j : &kScanPad);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = jb + u * 256 + t;
    if (j > j1) break;
    const uint4 c = j == j1 ? last : v[u];
    const int lo = (int)max(row0 - 16 * j, (int64_t)0), hi = (int)min(end - 16 * j, (int64_t)16);
    const uint64_t m0 = nz_bytes(c.x, c.y) & bytes_below(hi) & ~bytes_below(lo);
    const uint64_t m1 = nz_bytes(c.z, c.w) & bytes_below(hi - 8) & ~bytes_below(lo - 8);
    if (m0 | m1) {
      const int i = m0 ? __builtin_ctzll(m0) >> 3 : 8 + (__builtin_ctzll(m1) >> 3);
      return (int)(16 * j + i - row0);
    }
  }
  return INT_MAX;
}

__device__ int first_valid_row(const uint8_t* __restrict__ valid, int64_t row0, int T,
                               int* s_first) {
  const int t = threadIdx.x;
  if (t == 0) *s_first = INT_MAX;
  __syncthreads();
  if (T <= 0) return -1;
  const int64_t end = row0 + T;
  const int64_t j0 = row0 >> 4, j1 = (end - 1) >> 4;  // chunks holding the request's bytes
  uint8_t lb[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lb[i] = valid[min(16 * j1 + i, end - 1)];
  uint32_t lw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
    lw[w] = lb[4 * w] | lb[4 * w + 1] << 8 | lb[4 * w + 2] << 16 | (uint32_t)lb[4 * w + 3] << 24;
  const uint4 last = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  const uint4* vc = (const uint4*)valid;
  for (int64_t jb = j0; jb <= j1;) {
    const bool first = jb == j0;
    const int found = first ? scan_round<1>(vc, jb, j1, last, row0, end)
                            : scan_round<4>(vc, jb, j1, last, row0, end);
    jb += first ? 256 : 256 * 4;
    if (found != INT_MAX) atomicMin(s_first, found);
    __syncthreads();
    const int cur = *s_first;
    __syncthreads();
    if (cur != INT_MAX) break;
  }
  const int f = *s_first;
  return f == INT_MAX ? -1 : f;
}

// Read in place of ln_w / ln_b when there is no LayerNorm (values unused;
// global, not constant, memory, so the loads stay plain global loads).
__device__ float kNoLn[256];

constexpr int kGateSlice = 128;  // K per gate partial
constexpr int kGateRows = 16;    // gate rows per partial workgroup

// Split-K head-gate work riding in a compression launch.
struct GateArgs {
  const float* hidden;  // [M, K] f32
  const float* W;       // [K, N] f32
  float* part;          // [M, nslices, N] f32: part[m][s] = hidden[m, slice s] @ W[slice s, :]
  int M, K, N, nslices, nwg;  // nwg = nslices * ceil(M / 16); 0 = no gate work
};

// part[m][sl][n] for the 16 rows of tile mt, K slice sl; k added in order.
__device__ void gate_partial(const GateArgs& ga, int g) {
  __shared__ __attribute__((aligned(16))) float s_h[kGateRows][kGateSlice + 4];
  __shared__ __attribute__((aligned(16))) float s_w[kGateSlice][16];
  const int t = threadIdx.x;
  const int sl = g % ga.nslices, m0 = (g / ga.nslices) * kGateRows;
  const int k0 = sl * kGateSlice;
  const int M = ga.M, K = ga.K, N = ga.N;
  // hidden tile: row t/16, eight columns from 8*(t%16); rows past M clamped
  {
    const int hr = t >> 4, hc = (t & 15) * 8;
    const float* hp = ga.hidden + (int64_t)min(m0 + hr, M - 1) * K + k0 + hc;
    const float4 a = *(const float4*)hp, b = *(const float4*)(hp + 4);
    float4* dst = (float4*)&s_h[hr][hc];
    dst[0] = a;
    dst[1] = b;
  }
  // W tile: k row t/2, eight outputs from 8*(t%2); outputs past N are zero
  {
    const int kr = t >> 1, n0 = (t & 1) * 8;
    const float* wp = ga.W + (int64_t)(k0 + kr) * N;
    float v[8];
    if (N == 16) {
      const float4 a = *(const float4*)(wp + n0), b = *(const float4*)(wp + n0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = wp[min(n0 + j, N - 1)];
        v[j] = n0 + j < N ? x : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_w[kr][n0 + j] = v[j];
  }
  __syncthreads();
  const int m = t >> 4, n = t & 15;
  float acc = 0.f;
#pragma unroll 8
  for (int k = 0; k < kGateSlice; k += 4) {
    const float4 h = *(const float4*)&s_h[m][k];
    acc = fmaf(h.x, s_w[k][n], acc);
    acc = fmaf(h.y, s_w[k + 1][n], acc);
    acc = fmaf(h.z, s_w[k + 2][n], acc);
    acc = fmaf(h.w, s_w[k + 3][n], acc);
  }
  if (m0 + m < M && n < N) ga.part[((int64_t)(m0 + m) * ga.nslices + sl) * N + n] = acc;
}

// A whole decode step's start in the compression launch (dsa_gate_compress_live):
// the geometry from the live lengths, the store of the staged indexer row, and
// the recompression of the pool that row completes, which takes the row from
// registers rather than re-reading what this launch stores.
struct LiveArgs {
  const uint16_t* k_new;     // [B, D] staged rows; NULL: not a live call
  const uint16_t* gate_new;  // [B, D]
  int store_ln;              // normalise the stored k row (the per-token k_normed form)
  const float* sln_w;        // [D] LayerNorm of the stored row
  const float* sln_b;
  int32_t* q_req;            // [B] outputs of the geometry
  int32_t* q_pos;
  int32_t* new_from;
};

template <int LPP, int KP>  // lanes per pool = D / 8; pool slots
__global__ __launch_bounds__(256) void kpool_compress_kernel(
    uint16_t* __restrict__ k, uint16_t* __restrict__ gate,  // (written by a live call only)
    const uint16_t* __restrict__ ape, uint8_t* __restrict__ valid,
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ pool_off,
    const int32_t* __restrict__ live_len, int has_live, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, float eps,
    const int32_t* __restrict__ new_from, int pools_per_wg, int spec_pools,
    uint16_t* __restrict__ keys,
    int32_t* __restrict__ pool_start, uint8_t* __restrict__ pool_valid,
    int32_t* __restrict__ n_pools, int B, GateArgs ga, LiveArgs la) {
  constexpr int D = LPP * 8;
  constexpr int kpool = KP;
  constexpr int kGroups = 256 / LPP;  // pools in flight per workgroup
  __shared__ int s_first;
  if ((int)blockIdx.y >= B) {  // head-gate workgroups of the fused launch
    const int g = (blockIdx.y - B) * gridDim.x + blockIdx.x;
    if (g < ga.nwg) gate_partial(ga, g);
    return;
  }
  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int li = t % LPP;     // lane within the pool's lane group
  const int grp = t / LPP;    // pool group within the workgroup
  const int c0 = li * 8;      // first channel of this lane
  const bool live_call = la.k_new != nullptr;
  // The geometry loads, issued together (the empty asm keeps the compiler
  // from moving the live-length load into a branch of its own); the loads
  // that need no geometry go out with them.
  int g_lo = tok_off[r], g_hi = tok_off[r + 1], g_pb = pool_off[r], g_pe = pool_off[r + 1];
  int live = live_len[r];  // (tok_off when there are no live lengths)
  int g_nf = *(new_from ? new_from + r : tok_off + r);
  asm volatile("" : "+s"(g_lo), "+s"(g_hi), "+s"(g_pb), "+s"(g_pe), "+s"(live), "+s"(g_nf));
  const int64_t row0 = g_lo;
  const int region = g_hi - g_lo;
  const int n_live = max(live, 0);
  const int T = has_live ? min(n_live, region) : region;
  const int64_t pbase = g_pb;
  const int cap = g_pe - g_pb;
  // a live call writes row n_live - 1 and recompresses from it
  const int nf = live_call ? max(n_live - 1, 0) : new_from ? g_nf : 0;
  const bool incremental = live_call || new_from != nullptr;
  // the staged row (every lane loads its channels; one lane group uses them)
  const uint4 kst = *(const uint4*)(live_call ? la.k_new + (int64_t)r * D + c0 : ape + c0);
  const uint4 gst = *(const uint4*)(live_call ? la.gate_new + (int64_t)r * D + c0 : ape + c0);
  const bool post_ln = ln_w != nullptr;
  const float* lwp = post_ln ? ln_w : kNoLn;
  const float* lbp = post_ln ? ln_b : kNoLn;
  float lw[8], lb[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    lw[c] = lwp[c0 + c];
    lb[c] = lbp[c0 + c];
  }
  uint4 ap[KP];
#pragma unroll
  for (int s = 0; s < KP; ++s) ap[s] = *(const uint4*)(ape + s * D + c0);

  // One pool: slot softmax per channel, pooling, LayerNorm, one bf16 rounding.
  auto pool_out = [&](int p, int f, const uint4 (&kr)[KP], const uint4 (&gr)[KP], int allv) {
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int word = c >> 1, sh = (c & 1) * 16;
      float g[KP];
      float m = -INFINITY;
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const uint32_t gw = u4_word(gr[s], word), aw = u4_word(ap[s], word);
        g[s] = bf16_to_f32((gw >> sh) & 0xffffu) + bf16_to_f32((aw >> sh) & 0xffffu);
        m = fmaxf(m, g[s]);
      }
      float z = 0.f, acc = 0.f;
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const float e = expf(g[s] - m);
        z += e;
        const uint32_t kw = u4_word(kr[s], word);
        acc = fmaf(e, bf16_to_f32((kw >> sh) & 0xffffu), acc);
      }
      x[c] = acc / z;
    }
    uint4 key;
    if (!post_ln) {
      uint32_t pk[4];
#pragma unroll
      for (int c = 0; c < 8; c += 2) pk[c >> 1] = pack_bf16x2(x[c], x[c + 1]);
      key = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
      key = layer_norm8_bf16<LPP>(x, lw, lb, eps);
    }
    *(uint4*)(keys + (pbase + p) * D + c0) = key;
    if (li == 0) {
      pool_start[pbase + p] = f + p * kpool;
      pool_valid[pbase + p] = (uint8_t)allv;
    }
  };
  // The kpool rows from row0 + rs: all loads issued together; the validity
  // bytes are consumed at once (so no later instruction waits on them alone).
  auto load_rows = [&](const uint16_t* kb, const uint16_t* gb, const uint8_t* vbp, int64_t rs,
                       uint4 (&kr)[KP], uint4 (&gr)[KP], bool last_valid = false) {
    uint8_t vb[KP];
#pragma unroll
    for (int s = 0; s < KP; ++s) {
      kr[s] = *(const uint4*)(kb + (rs + s) * D + c0);
      gr[s] = *(const uint4*)(gb + (rs + s) * D + c0);
      vb[s] = vbp[rs + s];
    }
    int allv = 1;
#pragma unroll
    for (int s = 0; s < KP; ++s) allv &= (s == KP - 1 && last_valid) || vb[s] != 0;
    return allv;
  };

  if (!incremental) {
    // full mode: every slot of the request, in ascending order
    const int f = first_valid_row(valid, row0, T, &s_first);
    int P = f < 0 ? 0 : (T - f) / kpool;
    if (P > cap) P = cap;
    if (blockIdx.x == 0 && t == 0) n_pools[r] = P;
    const int s0 = blockIdx.x * pools_per_wg;
    const int s1 = min(cap, s0 + pools_per_wg);
    for (int p = s0 + grp; p < s1; p += kGroups) {
      if (p >= P) {  // sentinel slot past the full pools
        *(uint4*)(keys + (pbase + p) * D + c0) = make_uint4(0, 0, 0, 0);
        if (li == 0) {
          pool_start[pbase + p] = -1;
          pool_valid[pbase + p] = 0;
        }
        continue;
      }
      uint4 kr[KP], gr[KP];
      const int allv = load_rows(k, gate, valid, row0 + f + (int64_t)p * kpool, kr, gr);
      pool_out(p, f, kr, gr, allv);
    }
    return;
  }

  // Incremental mode: the pools holding a row at or after new_from are
  // rewritten, walked from the last pool down (group grp of workgroup x takes
  // the (x*pools_per_wg + grp)-th pool from the end).  In decode the newest
  // row creates work only when it completes a pool, and then the pools end
  // exactly at row T; so the rows of this group's pool under that alignment
  // load right away, before the first valid row f is known.  f itself comes
  // from slot 0 of the earlier call (the start of pool 0) when that slot holds
  // a pool starting before new_from -- rows before new_from are unchanged, so
  // f is too -- and from the scan otherwise.
  //
  // A live call also stores the staged row at nf (group 0 of the request's
  // first workgroup) and, when that row is the newest live row, uses it from
  // registers as the last slot of the pool ending at T.
  const int i0 = blockIdx.x * pools_per_wg + grp;
  const bool spec = i0 < spec_pools && T >= kpool * (i0 + 1);
  const int64_t srs = spec ? row0 + T - (int64_t)kpool * (i0 + 1) : 0;
  const bool subst = live_call && n_live >= 1 && nf == T - 1;  // the stored row is live row T-1
  const int fc = *(cap > 0 ? pool_start + pbase : tok_off + r);  // (unused when cap == 0)
  uint4 skr[KP], sgr[KP];
  // (with no such rows the loads read ape's kpool rows)
  const int sallv = load_rows(spec ? k : ape, spec ? gate : ape,
                              spec ? valid : (const uint8_t*)ape, srs, skr, sgr,
                              subst && i0 == 0);
  if (live_call) {
    uint4 kout = kst;
    if (la.store_ln) {  // (all lanes: the group sums need every lane of the group)
      float x[8], sw[8], sb[8];
      bf16x8_to_f32(kst, x);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sw[c] = la.sln_w[c0 + c];
        sb[c] = la.sln_b[c0 + c];
      }
      kout = layer_norm8_bf16<LPP>(x, sw, sb, eps);
    }
    if (blockIdx.x == 0 && grp == 0 && nf < region) {
      const int64_t row = row0 + nf;
      *(uint4*)(k + row * D + c0) = kout;
      *(uint4*)(gate + row * D + c0) = gst;
      if (li == 0) valid[row] = 1;
    }
    if (blockIdx.x == 0 && t == 0) {
      la.q_req[r] = r;
      la.q_pos[r] = n_live - 1;
      la.new_from[r] = nf;
    }
    if (subst && i0 == 0) {
      skr[KP - 1] = kout;
      sgr[KP - 1] = gst;
    }
  }
  const bool cached = cap > 0 && fc >= 0 && fc < nf;
  int f = cached ? fc : first_valid_row(valid, row0, T, &s_first);
  if (subst && !cached) f = f >= 0 ? min(f, T - 1) : T - 1;  // (row T-1 is valid now)
  int P = f < 0 ? 0 : (T - f) / kpool;
  if (P > cap) P = cap;
  if (blockIdx.x == 0 && t == 0) n_pools[r] = P;
  const int lo = (f >= 0 && nf >= f) ? min(P, (nf - f) / kpool) : 0;
  const bool aligned = f >= 0 && (T - f) % kpool == 0;
  for (int i = i0, j = 0; j * kGroups < pools_per_wg; ++j, i += kGroups) {
    const int p = P - 1 - i;
    if (p < lo) break;
    if (j == 0 && aligned) {
      pool_out(p, f, skr, sgr, sallv);
    } else {
      uint4 kr[KP], gr[KP];
      const int allv = load_rows(k, gate, valid, row0 + f + (int64_t)p * kpool, kr, gr);
      pool_out(p, f, kr, gr, allv);
    }
  }
}

}  // namespace

namespace {

dsa_status check_compress_args(int B, int D, int kpool, int max_cap, const int32_t* new_from,
                               int max_new, float eps, const float* ln_w, const float* ln_b) {
  DSA_REQUIRE(kpool >= 1 && kpool <= DSA_MAX_KPOOL, DSA_ERR_INVALID_ARG,
              "dsa_kpool_compress: kpool=%d outside [1,%d] (larger pools are refused, never "
              "truncated)",
              kpool, DSA_MAX_KPOOL);
  DSA_REQUIRE(D == 32 || D == 64 || D == 128 || D == 256, DSA_ERR_UNSUPPORTED,
              "dsa_kpool_compress: D=%d not in {32,64,128,256}", D);
  DSA_REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "dsa_kpool_compress: B=%d < 0", B);
  DSA_REQUIRE(max_cap >= 0, DSA_ERR_INVALID_ARG, "dsa_kpool_compress: max_cap=%d < 0", max_cap);
  DSA_REQUIRE(!new_from || max_new >= 1, DSA_ERR_INVALID_ARG,
              "dsa_kpool_compress: max_new=%d < 1 with new_from", max_new);
  DSA_REQUIRE(eps >= 0.f, DSA_ERR_INVALID_ARG, "dsa_kpool_compress: eps < 0");
  DSA_REQUIRE((ln_w == nullptr) == (ln_b == nullptr), DSA_ERR_INVALID_ARG,
              "dsa_kpool_compress: ln_w and ln_b must both be given or both be NULL");
  return DSA_OK;
}

// One launch: B rows of compression workgroups, then ga.nwg gate workgroups.
// k, gate and valid are written only by a live call (la.k_new set).
dsa_status launch_compress(const uint16_t* k, const uint16_t* gate, const uint16_t* ape,
                           const uint8_t* valid, const int32_t* tok_off, const int32_t* pool_off,
                           const int32_t* seq_len, const float* ln_w, const float* ln_b,
                           float eps, int B, int D, int kpool, int max_cap,
                           const int32_t* new_from, int max_new, uint16_t* keys,
                           int32_t* pool_start, uint8_t* pool_valid, int32_t* n_pools,
                           const GateArgs& ga, hipStream_t stream, const char* who,
                           const LiveArgs& la = LiveArgs{}) {
  const int lpp = D / 8;
  const int groups = 256 / lpp;
  int ppw, nx, spec = 0;
  if (new_from || la.k_new) {
    const int touch = (max_new + kpool - 1) / kpool;  // pools one request can touch
    ppw = groups;
    nx = (touch + ppw - 1) / ppw;
    spec = touch;
  } else {
    ppw = groups * 4;
    nx = (max_cap + ppw - 1) / ppw;
  }
  if (nx < 1) nx = 1;  // n_pools is written even with no slots
  const int gate_rows = (ga.nwg + nx - 1) / nx;
  DSA_REQUIRE((long long)B + gate_rows <= 65535, DSA_ERR_UNSUPPORTED,
              "%s: B=%d requests (+%d head-gate rows) above the 65535-row launch grid", who, B,
              gate_rows);
  dim3 grid(nx, B + gate_rows);
  if (dsa::trace_enabled())
    fprintf(stderr,
            "[dsa] %s B=%d D=%d kpool=%d max_cap=%d inc=%d gate_wg=%d grid=(%d,%d)\n", who, B,
            D, kpool, max_cap, new_from != nullptr || la.k_new != nullptr, ga.nwg, grid.x, grid.y);
#define DSA_LAUNCH_KP(LPP, KP)                                                                 \
  kpool_compress_kernel<LPP, KP><<<grid, 256, 0, stream>>>(                                     \
      const_cast<uint16_t*>(k), const_cast<uint16_t*>(gate), ape, const_cast<uint8_t*>(valid),  \
      tok_off, pool_off, seq_len ? seq_len : tok_off, seq_len != nullptr, ln_w, ln_b, eps,      \
      new_from, ppw, spec, keys, pool_start, pool_valid, n_pools, B, ga, la)
#define DSA_LAUNCH_KP_D(KP)            \
  switch (lpp) {                       \
    case 4: DSA_LAUNCH_KP(4, KP); break;   \
    case 8: DSA_LAUNCH_KP(8, KP); break;   \
    case 16: DSA_LAUNCH_KP(16, KP); break; \
    default: DSA_LAUNCH_KP(32, KP); break; \
  }
  if (dsa::dry_run()) return DSA_OK;
  switch (kpool) {
    case 1: DSA_LAUNCH_KP_D(1); break;
    case 2: DSA_LAUNCH_KP_D(2); break;
    case 3: DSA_LAUNCH_KP_D(3); break;
    case 4: DSA_LAUNCH_KP_D(4); break;
    case 5: DSA_LAUNCH_KP_D(5); break;
    case 6: DSA_LAUNCH_KP_D(6); break;
    case 7: DSA_LAUNCH_KP_D(7); break;
    default: DSA_LAUNCH_KP_D(8); break;
  }
#undef DSA_LAUNCH_KP_D
#undef DSA_LAUNCH_KP
  return dsa::check_launch(who);
}

// K slices of the split head-gate, or 1 when the dense head-gate call serves
// (then the "partials" buffer holds w itself).
int gate_slices(int M, int K) {
  if (M >= 1 && M <= 64 && K >= kGateSlice && K % kGateSlice == 0 && K / kGateSlice <= 64)
    return K / kGateSlice;
  return 1;
}

}  // namespace

DSA_EXPORT dsa_status dsa_kpool_compress(const uint16_t* k, const uint16_t* gate,
                                         const uint16_t* ape, const uint8_t* valid,
                                         const int32_t* tok_off, const int32_t* pool_off,
                                         const int32_t* seq_len, const float* ln_w,
                                         const float* ln_b, float eps, int B, int D, int kpool,
                                         int max_cap, const int32_t* new_from, int max_new,
                                         uint16_t* keys, int32_t* pool_start,
                                         uint8_t* pool_valid, int32_t* n_pools,
                                         hipStream_t stream) {
  const dsa_status st =
      check_compress_args(B, D, kpool, max_cap, new_from, max_new, eps, ln_w, ln_b);
  if (st != DSA_OK) return st;
  if (B == 0) return DSA_OK;
  DSA_REQUIRE(k && gate && ape && valid && tok_off && pool_off && keys && pool_start &&
                  pool_valid && n_pools,
              DSA_ERR_INVALID_ARG, "dsa_kpool_compress: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_kpool_compress", k, gate, ape, valid, tok_off, pool_off, seq_len, ln_w,
                      ln_b, new_from, keys, pool_start, pool_valid, n_pools);
  return launch_compress(k, gate, ape, valid, tok_off, pool_off, seq_len, ln_w, ln_b, eps, B, D,
                         kpool, max_cap, new_from, max_new, keys, pool_start, pool_valid,
                         n_pools, GateArgs{}, stream, "dsa_kpool_compress");
}

DSA_EXPORT int dsa_gate_split_count(int M, int K, int N) {
  if (M < 0 || K < 1 || N < 1 || N > DSA_MAX_INDEX_HEADS) return 0;
  return gate_slices(M, K);
}

DSA_EXPORT size_t dsa_gate_compress_workspace_size(int M, int K, int N) {
  const int ns = dsa_gate_split_count(M, K, N);
  if (ns < 1 || M < 1) return 0;
  return (size_t)ns * M * N * sizeof(float);
}

DSA_EXPORT dsa_status dsa_gate_compress(const float* hidden, const float* W, int M, int K, int N,
                                        float* gate_part, size_t gate_part_bytes,
                                        const uint16_t* k, const uint16_t* gate,
                                        const uint16_t* ape, const uint8_t* valid,
                                        const int32_t* tok_off, const int32_t* pool_off,
                                        const int32_t* seq_len, const float* ln_w,
                                        const float* ln_b, float eps, int B, int D, int kpool,
                                        int max_cap, const int32_t* new_from, int max_new,
                                        uint16_t* keys, int32_t* pool_start,
                                        uint8_t* pool_valid, int32_t* n_pools,
                                        hipStream_t stream) {
  DSA_REQUIRE(N >= 1 && N <= DSA_MAX_INDEX_HEADS, DSA_ERR_INVALID_ARG,
              "dsa_gate_compress: N=%d outside [1,%d]", N, DSA_MAX_INDEX_HEADS);
  DSA_REQUIRE(M >= 0 && K >= 1, DSA_ERR_INVALID_ARG, "dsa_gate_compress: M=%d K=%d", M, K);
  const dsa_status st =
      check_compress_args(B, D, kpool, max_cap, new_from, max_new, eps, ln_w, ln_b);
  if (st != DSA_OK) return st;
  const size_t need = dsa_gate_compress_workspace_size(M, K, N);
  DSA_REQUIRE(M == 0 || (gate_part && gate_part_bytes >= need), DSA_ERR_INVALID_ARG,
              "dsa_gate_compress: gate partials %zu bytes, need %zu", gate_part_bytes, need);
  DSA_REQUIRE(M == 0 || (hidden && W), DSA_ERR_INVALID_ARG,
              "dsa_gate_compress: NULL tensor pointer");
  DSA_REQUIRE(B == 0 || (k && gate && ape && valid && tok_off && pool_off && keys &&
                         pool_start && pool_valid && n_pools),
              DSA_ERR_INVALID_ARG, "dsa_gate_compress: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_gate_compress", hidden, W, gate_part, k, gate, ape, valid, tok_off,
                      pool_off, seq_len, ln_w, ln_b, new_from, keys, pool_start, pool_valid,
                      n_pools);
  const int ns = gate_slices(M, K);
  if (M > 0 && ns == 1) {  // dense head-gate: the partials buffer receives w
    const dsa_status g = dsa_head_gate(hidden, W, gate_part, M, K, N, nullptr, 0, stream);
    if (g != DSA_OK) return g;
    if (B == 0) return DSA_OK;
    return launch_compress(k, gate, ape, valid, tok_off, pool_off, seq_len, ln_w, ln_b, eps, B,
                           D, kpool, max_cap, new_from, max_new, keys, pool_start, pool_valid,
                           n_pools, GateArgs{}, stream, "dsa_gate_compress");
  }
  GateArgs ga{hidden, W, gate_part, M, K, N, ns, M > 0 ? ns * ((M + kGateRows - 1) / kGateRows) : 0};
  if (B == 0 && ga.nwg == 0) return DSA_OK;
  // with B == 0 the launch holds only gate workgroups (its compression
  // arguments are never read)
  return launch_compress(k, gate, ape, valid, tok_off, pool_off, seq_len, ln_w, ln_b, eps, B, D,
                         kpool, max_cap, new_from, max_new, keys, pool_start, pool_valid,
                         n_pools, ga, stream, "dsa_gate_compress");
}

DSA_EXPORT dsa_status dsa_gate_compress_live(
    const float* hidden, const float* W, int M, int K, int N, float* gate_part,
    size_t gate_part_bytes, uint16_t* k, uint16_t* gate, const uint16_t* ape, uint8_t* valid,
    const int32_t* tok_off, const int32_t* pool_off, const int32_t* seq_len,
    const uint16_t* k_new, const uint16_t* gate_new, const float* ln_w, const float* ln_b,
    int normed_rows, float eps, int B, int D, int kpool, int max_cap, uint16_t* keys,
    int32_t* pool_start, uint8_t* pool_valid, int32_t* n_pools, int32_t* q_req, int32_t* q_pos,
    int32_t* new_from, hipStream_t stream) {
  DSA_REQUIRE(N >= 1 && N <= DSA_MAX_INDEX_HEADS, DSA_ERR_INVALID_ARG,
              "dsa_gate_compress_live: N=%d outside [1,%d]", N, DSA_MAX_INDEX_HEADS);
  DSA_REQUIRE(M >= 0 && K >= 1, DSA_ERR_INVALID_ARG, "dsa_gate_compress_live: M=%d K=%d", M, K);
  const dsa_status st = check_compress_args(B, D, kpool, max_cap, nullptr, 1, eps, ln_w, ln_b);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(ln_w != nullptr, DSA_ERR_INVALID_ARG,
              "dsa_gate_compress_live: ln_w / ln_b are required (normed_rows selects where the "
              "LayerNorm applies)");
  const size_t need = dsa_gate_compress_workspace_size(M, K, N);
  DSA_REQUIRE(M == 0 || (gate_part && gate_part_bytes >= need), DSA_ERR_INVALID_ARG,
              "dsa_gate_compress_live: gate partials %zu bytes, need %zu", gate_part_bytes, need);
  DSA_REQUIRE(M == 0 || (hidden && W), DSA_ERR_INVALID_ARG,
              "dsa_gate_compress_live: NULL tensor pointer");
  DSA_REQUIRE(B == 0 || (k && gate && ape && valid && tok_off && pool_off && seq_len && k_new &&
                         gate_new && keys && pool_start && pool_valid && n_pools && q_req &&
                         q_pos && new_from),
              DSA_ERR_INVALID_ARG, "dsa_gate_compress_live: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_gate_compress_live", hidden, W, gate_part, k, gate, ape, valid, tok_off,
                      pool_off, seq_len, k_new, gate_new, ln_w, ln_b, keys, pool_start, pool_valid,
                      n_pools, q_req, q_pos, new_from);
  const LiveArgs la{k_new, gate_new, normed_rows != 0, ln_w, ln_b, q_req, q_pos, new_from};
  const float* pw = normed_rows ? nullptr : ln_w;  // LayerNorm after pooling
  const float* pb = normed_rows ? nullptr : ln_b;
  const int ns = gate_slices(M, K);
  if (M > 0 && ns == 1) {  // dense head-gate: the partials buffer receives w
    const dsa_status g = dsa_head_gate(hidden, W, gate_part, M, K, N, nullptr, 0, stream);
    if (g != DSA_OK) return g;
    if (B == 0) return DSA_OK;
    return launch_compress(k, gate, ape, valid, tok_off, pool_off, seq_len, pw, pb, eps, B, D,
                           kpool, max_cap, nullptr, 1, keys, pool_start, pool_valid, n_pools,
                           GateArgs{}, stream, "dsa_gate_compress_live", la);
  }
  GateArgs ga{hidden, W, gate_part, M, K, N, ns, M > 0 ? ns * ((M + kGateRows - 1) / kGateRows) : 0};
  if (B == 0 && ga.nwg == 0) return DSA_OK;
  return launch_compress(k, gate, ape, valid, tok_off, pool_off, seq_len, pw, pb, eps, B, D,
                         kpool, max_cap, nullptr, 1, keys, pool_start, pool_valid, n_pools, ga,
                         stream, "dsa_gate_compress_live", la);
}
