// a6: NoPE sparse MLA decode over the selected token ids.
//
// Atlas glm5next_dsa page: "Traps carried from Slice 8" (NoPE -- the 512-wide
// latent row is both key and value) and the MASKED_ATTN_MAX_KEYS note (a
// per-row gather of the selected ids is exactly the dense set-membership mask;
// the serving kernel keeps an online softmax and no full score row).
//
// Work split (flash-decoding): workgroup (chunk, 32-head block, query) covers
// one chunk of a query's selected ids for up to 32 heads; two workgroups share
// a compute unit (two waves per SIMD hide each other's latency), and the two
// head blocks of a chunk sit on the same XCD, so the second reads the rows
// from that XCD's L2.  The 4 waves of a workgroup split the 512 latent dims
// (128 each), not the heads:
//  * the chunk's ids are staged in LDS once; each wave loads its 128-dim slice
//    of the 32 gathered rows of a sub-chunk straight from HBM into the MFMA
//    A-operand layout, one sub-chunk ahead of the one it computes (a slot
//    with no id loads this query's own Q row, zeroed before use);
//  * QK^T: each wave computes the partial S^T[32 tok x 32 heads] over its dims
//    (v_mfma_f32_16x16x32_bf16, Q^T in registers); the partials meet in LDS
//    and wave w < 2 adds the four of head tile w in a fixed order, runs the
//    online softmax (log2 domain, reference max moved only when it grows by
//    more than 2^8) for those 16 heads, and publishes P in the PV A-operand
//    layout -- S^T's accumulator layout is that operand layout, with K index
//    8g+j of lane group g meaning token 4g+j (j < 4) or 16+4g+j-4;
//  * PV: O[32 heads x its 128 dims] += P . C_slice, the B operand read from
//    the wave's own slice in LDS (16 bytes = 8 dims per row per lane,
//    regrouped into 8 operands, so each lane owns 8 consecutive output dims).
// fp8 rows are widened to bf16 exactly in registers (the hardware conversion);
// the row scale multiplies the logits and the probabilities instead of the
// data.  With more than one chunk, per-chunk (max, sum) pairs and unnormalised
// O (bf16) go to the workspace and mla_combine_kernel merges them in chunk
// order.
//
// Paged cache (dsa_sparse_mla_decode_paged): the same kernel with the chunk's
// ids mapped to physical rows in the prologue.  The request's block-table row
// (up to kMaxBt entries) loads together with the ids and the Q rows and goes
// to LDS; each id then becomes page * page_rows + offset before it is staged,
// so the main loop is the flat kernel's.  Longer table rows read the entries
// past kMaxBt from memory.  Page numbers are clamped to the cache and block
// numbers to the table row, so no id can address memory outside them.
#include <limits.h>

#include <mutex>

#include "dsa_device.hpp"
#include "dsa_host.hpp"

// Workspace of dsa_sparse_mla_decode_noalloc: a fixed array in device memory,
// one per GPU the library runs on, held until the process ends.  In host code
// its name is only a host-side stand-in: kernels receive the device address
// that hipGetSymbolAddress returns for the current device (scratch_address).
static __device__ __align__(256) uint8_t scratch[DSA_MLA_SCRATCH_BYTES];

namespace {

using namespace dsa;

constexpr int L = DSA_KV_LORA;
constexpr int kSub = 32;                  // tokens per sub-chunk
constexpr int kSlice = 128;               // latent dims per wave
constexpr int kSliceRow = kSlice * 2 + 16;  // LDS bytes per token row of a slice (+pad)
constexpr int kHT = 2;                    // 16-head tiles per workgroup
constexpr int kHeadsWG = 16 * kHT;        // heads per workgroup
constexpr int kTargetWG = 512;            // aim for two workgroups per CU
// >= 64 ids per chunk: batches of few queries (one to four long-context
// requests) get up to twice as many workgroups with half the chain each
constexpr int kMinSubPerChunk = 2;
constexpr int kMaxTch = 2048;             // most ids per chunk
constexpr int kPF = 1;                    // sub-chunks of rows loading ahead of the one computed
constexpr int kMaxBt = 2048;              // block-table entries staged in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Chunking {
  int nchunks;
  int tch;  // ids per chunk (multiple of kSub)
};

Chunking mla_chunking(int Q, int Hm, int out_width) {
  const int nsub = (out_width + kSub - 1) / kSub;
  const int hb = (Hm + kHeadsWG - 1) / kHeadsWG;
  const long long base = (long long)Q * hb;
  long long want = (kTargetWG + base - 1) / base;
  const int max_chunks = nsub / kMinSubPerChunk > 1 ? nsub / kMinSubPerChunk : 1;
  if (want > max_chunks) want = max_chunks;
  const int min_chunks = (nsub * kSub + kMaxTch - 1) / kMaxTch;
  if (want < min_chunks) want = min_chunks;
  if (want < 1) want = 1;
  const int spc = (int)((nsub + want - 1) / want);
  return {(nsub + spc - 1) / spc, spc * kSub};
}

// (low halves of x and y) and (high halves), one v_perm_b32 each
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}
// 8 fp8 codes -> 8 bf16, in byte order, by the hardware conversion with a unit
// scale: exact (every E4M3 value, subnormals included, is a bf16 value); the
// NaN codes give NaN.  Word select 0 takes bytes 0-1 of a dword, 1 bytes 2-3.
__device__ __forceinline__ uint4 widen_fp8x8(uint2 v) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Read as the scale of a slot with no id (zero; global memory, so the load
// stays a plain global load).
__device__ float kNoScale;

template <bool FP8>
struct RowSlice;  // registers holding one lane's share of a sub-chunk's rows
template <>
struct RowSlice<false> {
  uint4 v[2][4];  // [token tile tt][k-step kk]: 8 bf16 dims
};
template <>
struct RowSlice<true> {
  uint2 v[2][4];  // 8 fp8 codes
};

// Where the rows live: flat (request r's row x at kv_off[r] + x) or paged.
struct CacheMap {
  const int32_t* kv_off;       // flat
  const int32_t* block_table;  // paged: [B, bt_stride]
  int bt_stride, page_rows, n_pages;
  int32_t* kvidx;              // paged, optional: [Q, out_width] physical rows
};

// ONE: the launch gives every query one chunk (the output is written here,
// no partials): only these instances carry the XCD-aware order and the
// non-temporal output stores, so the split launches' code stays as short
// as it was without them.
template <bool FP8, bool PAGED, bool ONE>
__global__ __launch_bounds__(256, 2) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ ckv_v,
    const float* __restrict__ ckv_scale, const CacheMap cm,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ tok, int Hm, int out_width,
    int tch, float sm_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int nq, int xcd_order) {
  __shared__ __attribute__((aligned(16))) uint8_t s_slice[4][kSub * kSliceRow];
  __shared__ f32x4_t s_exch[4][kHT][2][64];  // [source wave][head tile][token tile][lane]
  __shared__ uint4 s_p[kHT][64];             // P operands per head tile
  __shared__ float s_alpha[kHeadsWG];        // O rescale factor per head (when moved)
  __shared__ int s_moved[kHT];               // a head tile moved its reference max
  __shared__ __attribute__((aligned(16))) float s_mul[kSub];   // sm_scale*log2e*row scale
  __shared__ __attribute__((aligned(16))) float s_bias[kSub];  // 0, or -inf for no token
  __shared__ __attribute__((aligned(16))) float s_scl[kSub];   // row scale (1 for bf16)
  __shared__ float s_lrun[kHeadsWG];
  __shared__ int s_id[kMaxTch + kPF * kSub];  // the chunk's cache rows (-1: none)
  __shared__ int s_bt[PAGED ? kMaxBt : 1];  // the request's block-table row

  const int nchunks = gridDim.x;
  int chunk = blockIdx.x, hb = blockIdx.y, qx = blockIdx.z;
  if (ONE && xcd_order) {
    // XCD-aware order (the grid's queries padded to a multiple of 8):
    // workgroups go to the eight XCDs in turn, so ids eight apart share one;
    // every workgroup of query q takes an id on XCD q mod 8, so the second
    // head block re-reads the query's gathered rows from that XCD's L2.  The
    // padding workgroups leave at once.
    const int per_q = gridDim.x * gridDim.y;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int slot = lin >> 3, within = slot % per_q;
    qx = (slot / per_q) * 8 + (lin & 7);
    chunk = within % gridDim.x;
    hb = within / gridDim.x;
    if (qx >= nq) return;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int j0 = chunk * tch;
  const int j1 = min(out_width, j0 + tch);
  const int nsub = j1 > j0 ? (j1 - j0 + kSub - 1) / kSub : 0;
  const int32_t* trow = tok + (int64_t)qx * out_width;
  const int dim0 = w * kSlice;  // this wave's latent slice
  constexpr int kRowBytes = FP8 ? L : 2 * L;
  // Source of the loads for a token slot with no id: this query's own Q row
  // (always readable, at least one latent row long); the data is zeroed.
  const uint8_t* dummy = (const uint8_t*)(q + (int64_t)qx * Hm * L);

  // The chunk's ids (one per thread; longer chunks loop, rarely), the Q rows
  // and the request's first row are all in flight together; the ids then go
  // to LDS, and from there every later id is read, so no register loaded in
  // one sub-chunk is read in a later one except the latent rows.
  const int nid = nsub * kSub;
  const int r = q_req[qx];
  int id0 = trow[min(j0 + t, max(j1 - 1, 0))];

  // Q^T operand: qb[ht][kk] = Q[head hb*32 + ht*16 + col][dim0 + kk*32 + grp*8 .. +8].
  // Heads past Hm repeat head Hm-1: their softmax rows are computed and never
  // stored.
  bf16x8_t qb[kHT][4];
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht) {
    const int h = min(hb * kHeadsWG + ht * 16 + col, Hm - 1);
    const uint16_t* qrow = q + ((int64_t)qx * Hm + h) * L + dim0 + grp * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[ht][kk] = as_bf16x8(*(const uint4*)(qrow + kk * 32));
  }
  int64_t rowbase = 0;
  constexpr int kBtPerThread = PAGED ? kMaxBt / 256 : 1;
  int btv[kBtPerThread];
  const int32_t* btrow = nullptr;
  if constexpr (PAGED) {
    btrow = cm.block_table + (int64_t)r * cm.bt_stride;
#pragma unroll
    for (int k = 0; k < kBtPerThread; ++k) btv[k] = btrow[min(t + 256 * k, cm.bt_stride - 1)];
  } else {
    rowbase = cm.kv_off[r];
  }
  asm volatile("" ::: "memory");  // every load above is issued before any wait below
  if constexpr (PAGED) {
    asm volatile("" : "+v"(id0));  // loaded here, before the table's loads are waited for
#pragma unroll
    for (int k = 0; k < kBtPerThread; ++k) s_bt[t + 256 * k] = btv[k];
    __syncthreads();
    // logical id -> physical row; the optional index row is written once per
    // chunk (by the first head block)
    const unsigned pr = cm.page_rows;
    auto phys = [&](int id) {
      const unsigned b = (unsigned)id / pr, off = (unsigned)id - b * pr;
      const unsigned bc = min(b, (unsigned)cm.bt_stride - 1);
      const int pg = bc < (unsigned)kMaxBt ? s_bt[bc] : btrow[bc];
      return (int)(min((unsigned)pg, (unsigned)cm.n_pages - 1) * pr + off);
    };
    int32_t* krow = cm.kvidx && hb == 0 ? cm.kvidx + (int64_t)qx * out_width : nullptr;
    for (int i = t; i < nid + kPF * kSub; i += 256) {
      const int j = j0 + i;
      const int v = i < 256 ? id0 : trow[min(j, j1 - 1)];
      const int pv = j < j1 && v >= 0 ? phys(v) : -1;
      s_id[i] = pv;
      if (krow && j < j1) krow[j] = pv;
    }
  } else {
    // (entries from nid on are the -1 slots of the sub-chunks gathered past the end)
    s_id[t] = j0 + t < j1 ? id0 : -1;
    for (int i = t + 256; i < nid + kPF * kSub; i += 256) {
      const int j = j0 + i;
      const int v = trow[min(j, j1 - 1)];
      s_id[i] = j < j1 ? v : -1;
    }
  }
  __syncthreads();

  f32x4_t o[kHT][8];  // [head tile][e]: O[head ht*16 + grp*4 + i][dim0 + 8*col + e]
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[ht][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head w*16 + col (wave w < kHT owns head tile w)

  // a ring of kPF row sets: sub-chunk s is gathered into slot s mod kPF, kPF
  // sub-chunks ahead of its use; past the last sub-chunk every slot is empty
  // the zero scale's address, loaded once and kept in scalar registers: a
  // scalar load pending inside the loop would make every LDS wait a full one
  // (scalar loads return out of order)
  const float* zscl = &kNoScale;
  asm volatile("" : "+s"(zscl));
  RowSlice<FP8> ring[kPF];
  float rscl[kPF][2];  // row scales of tokens col, 16 + col (used by wave 0, lanes < 16)
  auto gather = [&](int s, RowSlice<FP8>& cr, float (&scl)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int id = s_id[s * kSub + tt * 16 + col];
      const uint8_t* src = id >= 0 ? (const uint8_t*)ckv_v + (rowbase + id) * kRowBytes : dummy;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int d = dim0 + kk * 32 + grp * 8;
        if (FP8)
          ((uint2*)cr.v[tt])[kk] = *(const uint2*)(src + d);
        else
          ((uint4*)cr.v[tt])[kk] = *(const uint4*)(src + 2 * d);
      }
      // the row scale (0 for no id) by a pointer select, so that nothing
      // consumes the loaded value here (a select on it would wait for every
      // load in flight, the rows just issued included)
      if (FP8) scl[tt] = *(id >= 0 ? ckv_scale + rowbase + id : zscl);
    }
  };
#pragma unroll
  for (int j = 0; j < kPF; ++j) {
    rscl[j][0] = rscl[j][1] = 1.f;
    gather(j, ring[j], rscl[j]);
  }

  uint8_t* my_slice = s_slice[w];
  auto body = [&](int s, RowSlice<FP8>& cr, float (&scl)[2]) {
    const int ida[2] = {s_id[s * kSub + col], s_id[s * kSub + 16 + col]};
    const bool live = __any(ida[0] >= 0 || ida[1] >= 0);  // uniform over the workgroup
    f32x4_t sacc[kHT][2];
    if (live) {
      // per-token logit multiplier and mask of this sub-chunk
      if (t < 16) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          s_mul[tt * 16 + t] = sm_log2 * scl[tt];
          s_bias[tt * 16 + t] = ida[tt] >= 0 ? 0.f : -INFINITY;
          s_scl[tt * 16 + t] = scl[tt];
        }
      }
      // partial S^T over this wave's dims, and the slice into LDS for PV
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) sacc[ht][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bool ok = ida[tt] >= 0;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          // the empty asm makes the loaded words opaque registers, so the
          // zeroing select stays a select (not a branch around the load)
          uint4 a;
          if (FP8) {
            uint2 raw = ((const uint2*)cr.v[tt])[kk];
            asm volatile("" : "+v"(raw.x), "+v"(raw.y));
            a = widen_fp8x8(ok ? raw : make_uint2(0, 0));
          } else {
            uint4 raw = ((const uint4*)cr.v[tt])[kk];
            asm volatile("" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z), "+v"(raw.w));
            a = ok ? raw : make_uint4(0, 0, 0, 0);
          }
          *(uint4*)(my_slice + (tt * 16 + col) * kSliceRow + (kk * 32 + grp * 8) * 2) = a;
#pragma unroll
          for (int ht = 0; ht < kHT; ++ht) sacc[ht][tt] = mfma16x16x32(as_bf16x8(a), qb[ht][kk], sacc[ht][tt]);
        }
      }
    }
    gather(s + kPF, cr, scl);  // later rows load while this sub-chunk computes
    if (live) {
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s_exch[w][ht][tt][lane] = sacc[ht][tt];
      __syncthreads();

      // wave w < kHT: full S^T of head tile w, softmax, P
      if (w < kHT) {
      float x[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4_t a0 = s_exch[0][w][tt][lane], a1 = s_exch[1][w][tt][lane];
        const f32x4_t a2 = s_exch[2][w][tt][lane], a3 = s_exch[3][w][tt][lane];
        const float4 mul = *(const float4*)(s_mul + tt * 16 + grp * 4);
        const float4 bias = *(const float4*)(s_bias + tt * 16 + grp * 4);
        const float mu[4] = {mul.x, mul.y, mul.z, mul.w};
        const float bi[4] = {bias.x, bias.y, bias.z, bias.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) x[tt * 4 + i] = fmaf(((a0[i] + a1[i]) + a2[i]) + a3[i], mu[i], bi[i]);
      }
      float mloc = x[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, x[k]);
      mloc = rows_max(mloc);
      const bool move = mloc > m_run + 8.f;
      // a head's first finite max only sets its reference (its O is still 0)
      const bool rescale = move && m_run != -INFINITY;
      const bool any_move = __any(rescale);
      if (any_move) {
        const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - mloc) : 1.f;
        l_run *= alpha;
        if (grp == 0) s_alpha[w * 16 + col] = alpha;
      }
      if (move) m_run = mloc;
      if (lane == 0) s_moved[w] = any_move;
      const bool none = m_run == -INFINITY;
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        p[k] = none ? 0.f : __builtin_amdgcn_exp2f(x[k] - m_run);
        psum += p[k];
      }
      l_run += rows_sum(psum);
      {
        uint32_t pw[4];
        float sc[8];
        if (FP8) {
          const float4 s0 = *(const float4*)(s_scl + grp * 4);
          const float4 s1 = *(const float4*)(s_scl + 16 + grp * 4);
          sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
          sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
        }
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const float p0 = FP8 ? p[k] * sc[k] : p[k], p1 = FP8 ? p[k + 1] * sc[k + 1] : p[k + 1];
          pw[k >> 1] = pack_bf16x2(p0, p1);
        }
        s_p[w][lane] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      }
      }
      __syncthreads();

      // rescale O where a head tile moved its reference max (rare)
      if (s_moved[0] | s_moved[kHT - 1]) {
#pragma unroll
        for (int ht = 0; ht < kHT; ++ht) {
          if (!s_moved[ht]) continue;
          float ai[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ai[i] = s_alpha[ht * 16 + grp * 4 + i];
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[ht][e][i] *= ai[i];
        }
      }
      // PV over this wave's slice
      bf16x8_t pa[kHT];
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht) pa[ht] = as_bf16x8(s_p[ht][lane]);
      uint4 u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = (j < 4 ? 0 : 16) + grp * 4 + (j & 3);
        u[j] = *(const uint4*)(my_slice + tk * kSliceRow + col * 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint32_t bw[4];
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
          const uint32_t a0 = u4_word(u[2 * m2], wd), a1 = u4_word(u[2 * m2 + 1], wd);
          bw[m2] = (e & 1) ? hi_pair(a0, a1) : lo_pair(a0, a1);
        }
        const bf16x8_t bv = as_bf16x8(make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
        for (int ht = 0; ht < kHT; ++ht) o[ht][e] = mfma16x16x32(pa[ht], bv, o[ht][e]);
      }
    }
  };
  for (int s0 = 0; s0 < nsub; s0 += kPF) {
#pragma unroll
    for (int j = 0; j < kPF; ++j)
      if (s0 + j < nsub) body(s0 + j, ring[j], rscl[j]);
  }

  // epilogue: per-head sums to every wave, then this wave's dims of all heads
  if (w < kHT && grp == 0) s_lrun[w * 16 + col] = l_run;
  __syncthreads();
  if (nchunks == 1) {
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hb * kHeadsWG + ht * 16 + grp * 4 + i;
        if (h >= Hm) continue;
        const float lv = s_lrun[ht * 16 + grp * 4 + i];
        const float inv = lv > 0.f ? 1.f / lv : 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) pk[e >> 1] = pack_bf16x2(o[ht][e][i] * inv, o[ht][e + 1][i] * inv);
        uint16_t* dst = out + ((int64_t)qx * Hm + h) * L + dim0 + col * 8;
        if constexpr (ONE) {
          // each output row is written once and read by no later workgroup:
          // a non-temporal store keeps it from evicting the latent rows, which
          // every query of a prefill batch gathers, from L2
          const u32x4_t v = {pk[0], pk[1], pk[2], pk[3]};
          __builtin_nontemporal_store(v, (u32x4_t*)dst);
        } else {
          *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      }
    const int hq = hb * kHeadsWG + w * 16 + col;
    if (lse && w < kHT && grp == 0 && hq < Hm)
      lse[(int64_t)qx * Hm + hq] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t pbase = ((int64_t)qx * nchunks + chunk) * Hm;
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hb * kHeadsWG + ht * 16 + grp * 4 + i;
        if (h >= Hm) continue;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) pk[e >> 1] = pack_bf16x2(o[ht][e][i], o[ht][e + 1][i]);
        // (non-temporal: the combine reads the partials once, from another
        // launch, so they need not stay in this XCD's L2)
        const u32x4_t v = {pk[0], pk[1], pk[2], pk[3]};
        __builtin_nontemporal_store(v, (u32x4_t*)(part_o + (pbase + h) * L + dim0 + col * 8));
      }
    const int hq = hb * kHeadsWG + w * 16 + col;
    if (w < kHT && grp == 0 && hq < Hm) {
      __builtin_nontemporal_store(m_run, part_ml + (pbase + hq) * 2);
      __builtin_nontemporal_store(l_run, part_ml + (pbase + hq) * 2 + 1);
    }
  }
}

// Merge the per-chunk partials of one (query, head) in chunk order; a wave per
// head, 8 dims per lane, HPW heads per workgroup (four, or one when the batch
// has too few queries to give every compute unit a four-head workgroup, so the
// partials stream through more compute units).  All chunks' loads of a
// batch are issued before any is used; the batch is the smallest of 4, 8, 16
// that holds every chunk (up to 16), so no load repeats a chunk needlessly.
// The partials are read, and the output written, non-temporally (each is
// touched once here; measured about a microsecond faster per decode step than
// plain accesses).
template <int kBatch, int HPW>
__global__ __launch_bounds__(256) void mla_combine_kernel(const uint16_t* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int nchunks, int Hm,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int h = blockIdx.x * HPW + (threadIdx.x >> 6), qx = blockIdx.y, lane = threadIdx.x & 63;
  if (h >= Hm) return;
  const int64_t b0 = (int64_t)qx * nchunks * Hm + h;
  // the running reference max M only grows: each batch rescales what came before
  float M = -INFINITY;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
    // lane k holds the (max, sum) pair of chunk c0 + k; the wave reads them
    // back one by one (one load per lane instead of one per chunk)
    const int cl = min(c0 + (lane & (kBatch - 1)), nchunks - 1);
    const float2 mlv = *(const float2*)(part_ml + (b0 + (int64_t)cl * Hm) * 2);
    uint4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = min(c0 + k, nchunks - 1);
      const int64_t pc = b0 + (int64_t)c * Hm;
      v[k] = __builtin_bit_cast(
          uint4, __builtin_nontemporal_load((const u32x4_t*)(part_o + pc * L + lane * 8)));
    }
    float2 ml[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      ml[k].x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv.x), k));
      ml[k].y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv.y), k));
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mb = c0 + k < nchunks ? fmaxf(Mb, ml[k].x) : Mb;
    if (Mb != M) {  // exp2(-inf) = 0 clears the (empty) history
      const float a = M == -INFINITY ? 0.f : exp2f(M - Mb);
      lsum *= a;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= a;
      M = Mb;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wgt = (M == -INFINITY || c0 + k >= nchunks) ? 0.f : exp2f(ml[k].x - M);
      lsum = fmaf(ml[k].y, wgt, lsum);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t word = u4_word(v[k], d >> 1);
        acc[d] = fmaf(wgt, bf16_to_f32((d & 1) ? (word >> 16) : (word & 0xffffu)), acc[d]);
      }
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint32_t pk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pk[k] = pack_bf16x2(acc[2 * k] * inv, acc[2 * k + 1] * inv);
  const u32x4_t ov = {pk[0], pk[1], pk[2], pk[3]};
  __builtin_nontemporal_store(ov, (u32x4_t*)(out + ((int64_t)qx * Hm + h) * L + lane * 8));
  if (lse && lane == 0)
    lse[(int64_t)qx * Hm + h] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

DSA_EXPORT size_t dsa_sparse_mla_decode_workspace_size(int Q, int Hm, int L_, int out_width,
                                                       int latent_dtype) {
  (void)latent_dtype;
  if (Q <= 0 || Hm <= 0 || out_width <= 0 || L_ != L) return 0;
  const Chunking ch = mla_chunking(Q, Hm, out_width);
  if (ch.nchunks <= 1) return 0;
  const size_t rows = (size_t)Q * ch.nchunks * Hm;
  // bf16 partial O rows, then (max, sum) f32 pairs (16-byte aligned)
  return rows * L * sizeof(uint16_t) + rows * 2 * sizeof(float);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch` per device (null: not yet)

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  The stream must belong to the
// current device: the address is that device's.
dsa_status scratch_address(hipStream_t stream, void** addr, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  DSA_REQUIRE(e == hipSuccess && dev >= 0 && dev < kMaxDevices, DSA_ERR_LAUNCH,
              "%s: hipGetDevice: %s (device %d)", who, hipGetErrorString(e), dev);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    DSA_REQUIRE(e == hipSuccess, DSA_ERR_INVALID_ARG, "%s: hipStreamGetDevice: %s", who,
                hipGetErrorString(e));
    DSA_REQUIRE(sdev == dev, DSA_ERR_INVALID_ARG,
                "%s: the stream belongs to device %d, the current device is %d", who, sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    DSA_REQUIRE(e == hipSuccess && p, DSA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch): %s",
                who, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return DSA_OK;
}


dsa_status launch_mla(const uint16_t* q, const void* ckv, const float* ckv_scale, int latent_dtype,
                      const CacheMap& cm, bool paged, const int32_t* q_req, const int32_t* tok,
                      int Q, int Hm, int L_, int out_width, float sm_scale, uint16_t* out,
                      float* lse, void* ws, size_t ws_bytes, hipStream_t stream, const char* who,
                      bool use_scratch = false) {
  DSA_REQUIRE(L_ == L, DSA_ERR_UNSUPPORTED,
              "%s: latent width L=%d, the kernels read exactly %d (a NoPE cache row is "
              "kv_lora_rank wide)",
              who, L_, L);
  DSA_REQUIRE(Hm >= 1, DSA_ERR_INVALID_ARG, "%s: Hm=%d < 1 (no heads)", who, Hm);
  DSA_REQUIRE(out_width >= 1, DSA_ERR_INVALID_ARG, "%s: out_width=%d < 1", who, out_width);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "%s: Q=%d < 0", who, Q);
  DSA_REQUIRE(latent_dtype == DSA_LATENT_BF16 || latent_dtype == DSA_LATENT_FP8_E4M3,
              DSA_ERR_INVALID_ARG, "%s: unknown latent dtype %d", who, latent_dtype);
  DSA_REQUIRE(latent_dtype != DSA_LATENT_FP8_E4M3 || ckv_scale, DSA_ERR_INVALID_ARG,
              "%s: fp8 latent without row scales", who);
  if (paged) {
    DSA_REQUIRE(cm.bt_stride >= 1 && cm.page_rows >= 1 && cm.n_pages >= 1, DSA_ERR_INVALID_ARG,
                "%s: bt_stride=%d, page_rows=%d, n_pages=%d (each must be >= 1)", who,
                cm.bt_stride, cm.page_rows, cm.n_pages);
    DSA_REQUIRE((long long)cm.n_pages * cm.page_rows <= INT_MAX, DSA_ERR_UNSUPPORTED,
                "%s: %d pages of %d rows exceed 2^31-1 cache rows", who, cm.n_pages,
                cm.page_rows);
  }
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(q && ckv && (paged ? cm.block_table != nullptr : cm.kv_off != nullptr) && q_req &&
                  tok && out,
              DSA_ERR_INVALID_ARG, "%s: NULL tensor pointer", who);
  DSA_REQUIRE_ALIGNED(who, q, ckv, ckv_scale, cm.kv_off, cm.block_table, cm.kvidx, q_req, tok, out,
                      lse, ws);
  const size_t need = dsa_sparse_mla_decode_workspace_size(Q, Hm, L_, out_width, latent_dtype);
  if (use_scratch) {  // the library's fixed array instead of a workspace argument
    DSA_REQUIRE(need <= (size_t)DSA_MLA_SCRATCH_BYTES, DSA_ERR_UNSUPPORTED,
                "%s: Q=%d Hm=%d out_width=%d need %zu bytes of workspace, above the library's "
                "fixed %zu (use dsa_sparse_mla_decode with a workspace)",
                who, Q, Hm, out_width, need, (size_t)DSA_MLA_SCRATCH_BYTES);
    ws = nullptr;
    ws_bytes = need;
    if (need > 0) {
      const dsa_status st = scratch_address(stream, &ws, who);
      if (st != DSA_OK) return st;
    }
  }
  DSA_REQUIRE(ws_bytes >= need && (need == 0 || ws), DSA_ERR_INVALID_ARG,
              "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
  const Chunking ch = mla_chunking(Q, Hm, out_width);
  uint16_t* part_o = need ? (uint16_t*)ws : nullptr;
  float* part_ml = need ? (float*)((uint16_t*)ws + (size_t)Q * ch.nchunks * Hm * L) : nullptr;
  // one chunk per query and at least 8 queries: the XCD-aware order (queries
  // padded to a multiple of 8), so the two head blocks of a query gather its
  // rows through one L2.  (With chunks, as at decode, the same order cut the
  // call's fetch from 42.3 to 34.9 MB at decode32k but made it slower, 21.8 ->
  // 22.4 us, so split calls keep the plain order.)
  const int xcd_order = ch.nchunks == 1 && Q >= 8 && (Q + 7) / 8 * 8 <= 65535;
  dim3 grid(ch.nchunks, (Hm + kHeadsWG - 1) / kHeadsWG, xcd_order ? (Q + 7) / 8 * 8 : Q);
  DSA_REQUIRE(grid.y <= 65535u && grid.z <= 65535u, DSA_ERR_UNSUPPORTED,
              "%s: Q=%d or Hm=%d outside the launch grid", who, Q, Hm);
  const float sm_log2 = sm_scale * kLog2e;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] %s Q=%d Hm=%d out_width=%d fp8=%d paged=%d chunks=%d tch=%d\n", who, Q,
            Hm, out_width, latent_dtype, (int)paged, ch.nchunks, ch.tch);
#define DSA_LAUNCH_MLA(F, P)                                                                 \
  if (ch.nchunks == 1)                                                                        \
    sparse_mla_kernel<F, P, true><<<grid, 256, 0, stream>>>(q, ckv, ckv_scale, cm, q_req, tok, \
                                                            Hm, out_width, ch.tch, sm_log2,   \
                                                            out, lse, part_o, part_ml, Q,     \
                                                            xcd_order);                       \
  else                                                                                        \
    sparse_mla_kernel<F, P, false><<<grid, 256, 0, stream>>>(q, ckv, ckv_scale, cm, q_req,    \
                                                             tok, Hm, out_width, ch.tch,      \
                                                             sm_log2, out, lse, part_o,       \
                                                             part_ml, Q, xcd_order)
  const bool fp8 = latent_dtype == DSA_LATENT_FP8_E4M3;
  if (dsa::dry_run()) return DSA_OK;
  if (paged) {
    if (fp8) DSA_LAUNCH_MLA(true, true);
    else DSA_LAUNCH_MLA(false, true);
  } else {
    if (fp8) DSA_LAUNCH_MLA(true, false);
    else DSA_LAUNCH_MLA(false, false);
  }
#undef DSA_LAUNCH_MLA
  dsa_status st = dsa::check_launch(who);
  if (st != DSA_OK || ch.nchunks == 1) return st;
  // four heads per workgroup while that fills the chip (256 compute units)
  const bool wide = (long long)Q * ((Hm + 3) / 4) >= 256;
  const int hpw = wide ? 4 : 1;
  const dim3 cgrid((Hm + hpw - 1) / hpw, Q);
#define DSA_LAUNCH_COMBINE(B)                                                                  \
  if (wide)                                                                                    \
    mla_combine_kernel<B, 4><<<cgrid, 256, 0, stream>>>(part_o, part_ml, ch.nchunks, Hm, out,  \
                                                        lse);                                  \
  else                                                                                         \
    mla_combine_kernel<B, 1><<<cgrid, 64, 0, stream>>>(part_o, part_ml, ch.nchunks, Hm, out, lse)
  if (ch.nchunks <= 4) DSA_LAUNCH_COMBINE(4);
  else if (ch.nchunks <= 8) DSA_LAUNCH_COMBINE(8);
  else DSA_LAUNCH_COMBINE(16);
#undef DSA_LAUNCH_COMBINE
  return dsa::check_launch(who);
}

}  // namespace

DSA_EXPORT dsa_status dsa_sparse_mla_decode(const uint16_t* q, const void* ckv,
                                            const float* ckv_scale, int latent_dtype,
                                            const int32_t* kv_off, const int32_t* q_req,
                                            const int32_t* tok, int Q, int Hm, int L_,
                                            int out_width, float sm_scale, uint16_t* out,
                                            float* lse, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  CacheMap cm{kv_off, nullptr, 0, 0, 0, nullptr};
  return launch_mla(q, ckv, ckv_scale, latent_dtype, cm, false, q_req, tok, Q, Hm, L_, out_width,
                    sm_scale, out, lse, ws, ws_bytes, stream, "dsa_sparse_mla_decode");
}


DSA_EXPORT dsa_status dsa_sparse_mla_decode_noalloc(const uint16_t* q, const void* ckv,
                                                    const float* ckv_scale, int latent_dtype,
                                                    const int32_t* kv_off, const int32_t* q_req,
                                                    const int32_t* tok, int Q, int Hm, int L_,
                                                    int out_width, float sm_scale, uint16_t* out,
                                                    float* lse, hipStream_t stream) {
  CacheMap cm{kv_off, nullptr, 0, 0, 0, nullptr};
  return launch_mla(q, ckv, ckv_scale, latent_dtype, cm, false, q_req, tok, Q, Hm, L_, out_width,
                    sm_scale, out, lse, nullptr, 0, stream, "dsa_sparse_mla_decode_noalloc",
                    /*use_scratch=*/true);
}

DSA_EXPORT dsa_status dsa_sparse_mla_decode_paged(
    const uint16_t* q, const void* ckv, const float* ckv_scale, int latent_dtype,
    const int32_t* block_table, int bt_stride, int page_rows, int n_pages, const int32_t* q_req,
    const int32_t* tok, int Q, int Hm, int L_, int out_width, float sm_scale, uint16_t* out,
    float* lse, int32_t* kvidx, void* ws, size_t ws_bytes, hipStream_t stream) {
  CacheMap cm{nullptr, block_table, bt_stride, page_rows, n_pages, kvidx};
  return launch_mla(q, ckv, ckv_scale, latent_dtype, cm, true, q_req, tok, Q, Hm, L_, out_width,
                    sm_scale, out, lse, ws, ws_bytes, stream, "dsa_sparse_mla_decode_paged");
}
