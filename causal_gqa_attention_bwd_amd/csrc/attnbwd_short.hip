// attnbwd_short.hip -- the short-sequence backward (attn_bwd_short): page
// "llm.istanbul -- 10_backward_attention.wgsl", kernels
// attention_backward_short and attention_backward_short_dKdV (the variant for
// sequences of at most 1024 positions).  Same sums as attn_bwd / attn_bwd_o:
//   P = exp(scale q.k - LSE), dP = dO.v, D = sum_j P dP (or dO.O),
//   dS = scale P (dP - D), dQ += sum_j dS k, dK += sum dS q, dV += sum P dO
// over the keys j with seg[s] <= j <= s, dK and dV summed over the KV group.
//
// At these lengths the long-sequence kernels are latency-bound: few tiles,
// each walking its keys (or queries) one 32-row block after another, over
// four launches.  Here one launch does the whole backward when the forward
// output O is given (the row term is then dO.O, formed where it is needed):
//   * workgroups of the key role own one 32-key block of one KV head: dK and
//     dV of those keys over every visible (query block, head of the group);
//   * workgroups of the query role own one 32-query block of one head: dQ of
//     those queries over every visible key block.
// Within a workgroup the visible blocks are dealt round-robin to the four
// waves, each of which sums its share in its own accumulators; the four
// partial sums are then added in wave order through LDS.  Every sum has one
// writer and a fixed order: deterministic, no atomics.  Without O, a first
// launch of the query role computes D = sum_j P dP into a workspace.  When a
// KV group's heads are many against the sequence, the key role's heads are
// split over several workgroups whose partial sums a last launch adds in
// split order (k_short_sum).
//
// Products: v_mfma_f32_32x32x2_f32.  Lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; register r of the 32x32 result holds row crow(r, l/32),
// column l%32.  A lane keeps one row's contraction columns of its half-wave
// (the contraction order over columns is free), so the score tiles come out
// with lane <-> query (query role: S^T = K Q^T) or lane <-> key (key role:
// S = Q K^T), and their registers are the A operands of the next products.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

#define SHORT_MAX_S 1024  // 32 blocks of 32: block sets fit one 32-bit mask

struct ShortArgs {
  const float *Q, *K, *V, *O, *dO, *LSE;  // O NULL: the row term is in Dws
  const uint32_t* seg;                     // NULL = all zeros
  float *dQ, *dK, *dV;
  float* Dws;  // [S, H] row term (written by the row-term launch when O is NULL)
  float* part; // ksplit > 1: [2 ksplit][S, KV, d] partial dK, dV of each head split
  int S, H, KV, d, nqb;
  int ksplit;  // workgroups sharing a key block's heads (a power of two dividing H / KV)
  float scale;
};

template <int DP>
struct ShortGeom {
  static constexpr int HD = DP / 2;   // contraction columns per half-wave
  static constexpr int LDT = DP + 4;  // LDS row pitch of a staged 32-row tile
  static constexpr int NC = DP / 32;  // 32-column output tiles
  static constexpr int LDS_FLOATS = 4 * 2 * 32 * LDT;  // two tiles per wave
};

// ---------------------------------------------------------------------------
// Loads.  Every global read goes through a buffer resource: an offset beyond
// the buffer (SHORT_OOB) reads zeros, so rows past the end, columns past d
// and item slots past a wave's last item need no branch, and the compiler
// can count the loads in flight exactly (a wave waits only for the item it
// is about to use, not for the next one's loads).
// ---------------------------------------------------------------------------
#define SHORT_OOB 0x80000000u  // beyond every buffer here (sizes are checked below 2^31)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float4 ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}
__device__ __forceinline__ float ld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Columns hf*HD .. hf*HD + HD - 1 of the row starting at element `row`
// (zeros beyond d, and everywhere when !ok).
template <int HD>
__device__ __forceinline__ void load_half(__amdgpu_buffer_rsrc_t r, size_t row, int hf, int d,
                                          bool ok, float* out) {
#pragma unroll
  for (int t = 0; t < HD; t += 4) {
    const int c = hf * HD + t;
    const uint32_t off = (ok && c < d) ? (uint32_t)((row + c) * 4) : SHORT_OOB;
    const float4 x = ld4(r, off);
    out[t] = x.x; out[t + 1] = x.y; out[t + 2] = x.z; out[t + 3] = x.w;
  }
}

template <int HD>
__device__ __forceinline__ void store_half(float* dst, const float* v) {
#pragma unroll
  for (int t = 0; t < HD; t += 4)
    *reinterpret_cast<float4*>(dst + t) = make_float4(v[t], v[t + 1], v[t + 2], v[t + 3]);
}

// OR of a 32-bit value over the wave.
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o);
  return x;
}

// The k-th set bit of m (k < popcount(m)).
__device__ __forceinline__ int nth_bit(uint32_t m, int k) {
  for (; k > 0; --k) m &= m - 1;
  return __builtin_ctz(m);
}

// The sequence's document starts into LDS, padded to whole blocks with ~0
// (a padding row sees no key), then a workgroup barrier.  Each role calls it
// after issuing the loads that do not depend on seg, so both are in flight
// together.
__device__ __forceinline__ void stage_seg(const ShortArgs& a, uint32_t* sSeg) {
  for (int i = threadIdx.x; i < 32 * a.nqb; i += 256)
    sSeg[i] = i < a.S ? (a.seg ? a.seg[i] : 0u) : 0xffffffffu;
  __syncthreads();
}

// The += write-back of a 32-row block: thread t owns elements t, t + 256, ...
// of the block's [32][DP] tile (row e / DP, column e % DP).  Their old values
// are read at the start of the workgroup and the new ones written at the end.
template <int DP>
struct BlockOut {
  static constexpr int N = 32 * DP / 256;
  float old[N];
  __device__ __forceinline__ uint32_t offset(int e, int r0, int S, int d, int heads, int head) const {
    const int row = e / DP, col = e % DP;
    return (r0 + row < S && col < d)
               ? (uint32_t)((((size_t)(r0 + row) * heads + head) * d + col) * 4)
               : SHORT_OOB;
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int r0, int S, int d, int heads,
                                       int head) {
#pragma unroll
    for (int n = 0; n < N; ++n)
      old[n] = ld1(r, offset(threadIdx.x + 256 * n, r0, S, d, heads, head));
  }
};

// ---------------------------------------------------------------------------
// Query role: dQ of query block qb, head h (ROWTERM: only D = sum_j P dP).
// A wave's items are the visible key blocks number wave, wave + 4, ...; the
// next item's K and V rows are loaded while the current item's later
// products run.
// ---------------------------------------------------------------------------
template <int DP, bool ROWTERM>
__device__ __forceinline__ void short_query(const ShortArgs& a, int qb, int h, float* lds,
                                            uint32_t* sSeg) {
  using G = ShortGeom<DP>;
  constexpr int HD = G::HD, LDT = G::LDT, NC = G::NC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H, d = a.d, g = H / a.KV, kvh = h / g;
  const int i0 = qb * 32, i = i0 + l32;
  const bool q_ok = i < S;
  const float sc2 = a.scale * ATTN_LOG2E;
  const size_t qbytes = (size_t)S * H * d * 4, kbytes = (size_t)S * a.KV * d * 4;
  const auto rQ = rsrc(a.Q, qbytes), rdO = rsrc(a.dO, qbytes);
  const auto rK = rsrc(a.K, kbytes), rV = rsrc(a.V, kbytes);

  float qB[HD], oB[HD];
  const size_t qrow = ((size_t)i * H + h) * d;
  load_half<HD>(rQ, qrow, hf, d, q_ok, qB);
  load_half<HD>(rdO, qrow, hf, d, q_ok, oB);
  const uint32_t roff = q_ok ? (uint32_t)(((size_t)i * H + h) * 4) : SHORT_OOB;
  const float lse2 = ld1(rsrc(a.LSE, (size_t)S * H * 4), roff) * ATTN_LOG2E;
  float Di = 0.f;
  BlockOut<DP> out;
  if constexpr (!ROWTERM) {
    if (a.O) {
      float ov[HD];
      load_half<HD>(rsrc(a.O, qbytes), qrow, hf, d, q_ok, ov);
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < HD; ++t) s = fmaf(oB[t], ov[t], s);
      Di = s + __shfl_xor(s, 32);
    } else {
      Di = ld1(rsrc(a.Dws, (size_t)S * H * 4), roff);
    }
    out.load(rsrc(a.dQ, qbytes), i0, S, d, H, h);
  }

  stage_seg(a, sSeg);
  const uint32_t si = sSeg[i];  // ~0 past the end
  // key blocks this query block sees: the union of [seg_i / 32, i / 32]
  uint32_t kmask = 0;
  if (q_ok && si <= (uint32_t)i)
    kmask = ((2u << (i >> 5)) - 1u) & ~((1u << (si >> 5)) - 1u);
  kmask = __builtin_amdgcn_readfirstlane(wave_or(kmask));
  const int nitems = __builtin_popcount(kmask);

  float* sK = lds + wave * 32 * LDT;  // this wave's K tile
  f32x16 acc[ROWTERM ? 1 : NC];
#pragma unroll
  for (int m = 0; m < (ROWTERM ? 1 : NC); ++m) acc[m] = zero16();
  float dsum = 0.f;

  // item k (k >= nitems: an empty slot whose loads read zeros)
  auto issue = [&](int k, float* kA, float* vA) {
    const bool ok = k < nitems;
    const int j0 = 32 * nth_bit(kmask, ok ? k : 0);
    const size_t krow = ((size_t)(j0 + l32) * a.KV + kvh) * d;
    load_half<HD>(rK, krow, hf, d, ok && j0 + l32 < S, kA);
    load_half<HD>(rV, krow, hf, d, ok && j0 + l32 < S, vA);
  };
  // the item's K and V rows are read only by the score products: once they
  // are issued, the next item's loads go into the same registers
  float kA[HD], vA[HD];
  auto compute = [&](int k) {
    const int j0 = 32 * nth_bit(kmask, k);
    if constexpr (!ROWTERM) store_half<HD>(sK + l32 * LDT + hf * HD, kA);
    // S^T = K Q^T and dP^T = V dO^T: register r <-> key crow(r, hf), lane <-> query
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int t = 0; t < HD; ++t) {
      s = mfma32(kA[t], qB[t], s);
      dp = mfma32(vA[t], oB[t], dp);
    }
    issue(k + 4, kA, vA);  // in flight during the rest of this item
    // the dQ product's B operands (K from the tile) are read while the
    // probabilities are formed
    float kb[ROWTERM ? 1 : 16][NC];
    if constexpr (!ROWTERM) {
      __builtin_amdgcn_wave_barrier();  // the wave's K rows are in LDS (in-order LDS)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) kb[r][c] = sK[crow(r, hf) * LDT + l32 + 32 * c];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + crow(r, hf);
      const bool vis = q_ok && (uint32_t)j >= si && j <= i;
      // computed unconditionally and then selected: a masked entry's value
      // (possibly inf) is discarded, and the loop stays free of branches
      const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse2));
      const float p = vis ? e : 0.f;
      if constexpr (ROWTERM) dsum = fmaf(p, dp[r], dsum);
      else s[r] = p * (dp[r] - Di);  // dS / scale
    }
    if constexpr (!ROWTERM) {
      // dQ += dS K: A = dS^T registers (lane <-> query), B = K from the tile
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = mfma32(s[r], kb[r][c], acc[c]);
      __builtin_amdgcn_wave_barrier();
    }
  };
  issue(wave, kA, vA);
  for (int k = wave; k < nitems; k += 4) compute(k);

  __syncthreads();  // every wave is done with its tile: the LDS is the reduction buffer
  if constexpr (ROWTERM) {
    float* sR = lds;  // [4][32]
    const float tot = dsum + __shfl_xor(dsum, 32);
    if (hf == 0) sR[wave * 32 + l32] = tot;
    __syncthreads();
    if (tid < 32 && i0 + tid < S)
      a.Dws[(size_t)(i0 + tid) * H + h] =
          ((sR[tid] + sR[32 + tid]) + sR[64 + tid]) + sR[96 + tid];
  } else {
    float* sR = lds;  // [4][32][DP]: row crow(r, hf), column 32 c + l32
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) sR[(wave * 32 + crow(r, hf)) * DP + 32 * c + l32] = acc[c][r];
    __syncthreads();
#pragma unroll
    for (int n = 0; n < BlockOut<DP>::N; ++n) {
      const int e = tid + 256 * n, row = e / DP, col = e % DP;
      if (i0 + row < S && col < d) {
        const float t = ((sR[e] + sR[32 * DP + e]) + sR[64 * DP + e]) + sR[96 * DP + e];
        a.dQ[((size_t)(i0 + row) * H + h) * d + col] = out.old[n] + a.scale * t;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key role: dK and dV of key block kb, KV head kvh, over the heads of head
// split `split` (all of the group's heads when ksplit = 1).  A wave's items
// are numbers wave, wave + 4, ... of the (visible query block, head of the
// split) pairs, query block major; the next item's Q, dO (and O) rows are
// loaded while the current item's later products run.  With one split the
// workgroup adds its sums into dK, dV; with several it writes them to its
// split's slices of `part`, which k_short_sum adds in split order.
// ---------------------------------------------------------------------------
template <int HD>
struct KeyItem {
  float q[HD], o[HD], fo[HD];  // the lane's halves of Q, dO, O (row i0 + l32)
  float lse, dws;              // that row's LSE and (without O) D
};

template <int DP>
__device__ __forceinline__ void short_key(const ShortArgs& a, int kb, int kvh, int split,
                                          float* lds, float* sRow, uint32_t* sSeg) {
  using G = ShortGeom<DP>;
  constexpr int HD = G::HD, LDT = G::LDT, NC = G::NC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H, d = a.d, g = H / a.KV;
  const int gs = g / a.ksplit, head0 = kvh * g + split * gs;  // this split's heads
  const int j0 = kb * 32, j = j0 + l32;
  const bool k_ok = j < S;
  const float sc2 = a.scale * ATTN_LOG2E;
  const size_t qbytes = (size_t)S * H * d * 4, kbytes = (size_t)S * a.KV * d * 4;
  const auto rQ = rsrc(a.Q, qbytes), rdO = rsrc(a.dO, qbytes);
  const auto rO = rsrc(a.O, a.O ? qbytes : 0);
  const auto rL = rsrc(a.LSE, (size_t)S * H * 4), rD = rsrc(a.Dws, a.Dws ? (size_t)S * H * 4 : 0);

  float kB[HD], vB[HD];
  const size_t krow = ((size_t)j * a.KV + kvh) * d;
  load_half<HD>(rsrc(a.K, kbytes), krow, hf, d, k_ok, kB);
  load_half<HD>(rsrc(a.V, kbytes), krow, hf, d, k_ok, vB);
  BlockOut<DP> outK, outV;
  if (a.ksplit == 1) {
    outK.load(rsrc(a.dK, kbytes), j0, S, d, a.KV, kvh);
    outV.load(rsrc(a.dV, kbytes), j0, S, d, a.KV, kvh);
  }

  stage_seg(a, sSeg);
  // query blocks with a row that sees a key of this block:
  // i >= j0, seg_i <= i and seg_i <= j0 + 31
  uint32_t qmask = 0;
  for (int i = j0 + lane; i < S; i += 64) {
    const uint32_t si = sSeg[i];
    if (si <= (uint32_t)i && si <= (uint32_t)(j0 + 31)) qmask |= 1u << (i >> 5);
  }
  qmask = __builtin_amdgcn_readfirstlane(wave_or(qmask));
  const int nitems = __builtin_popcount(qmask) * gs;

  float* sQ = lds + wave * 2 * 32 * LDT;  // this wave's Q and dO tiles
  float* sO = sQ + 32 * LDT;
  float* sL = sRow + wave * 64;  // LSE * log2e and D of the item's 32 rows
  float* sD = sL + 32;
  f32x16 accK[NC], accV[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) accK[c] = accV[c] = zero16();

  // item k: query block nth_bit(qmask, k / gs), head head0 + k % gs (k >=
  // nitems: an empty slot whose loads read zeros)
  auto issue = [&](int k, KeyItem<HD>& it) {
    const bool ok = k < nitems;
    const int kk = ok ? k : 0;
    const int i = 32 * nth_bit(qmask, kk / gs) + l32, h = head0 + kk % gs;
    const bool q_ok = ok && i < S;
    const size_t qrow = ((size_t)i * H + h) * d;
    load_half<HD>(rQ, qrow, hf, d, q_ok, it.q);
    load_half<HD>(rdO, qrow, hf, d, q_ok, it.o);
    if (a.O) load_half<HD>(rO, qrow, hf, d, q_ok, it.fo);
    const uint32_t roff = q_ok ? (uint32_t)(((size_t)i * H + h) * 4) : SHORT_OOB;
    it.lse = ld1(rL, roff);
    it.dws = a.O ? 0.f : ld1(rD, roff);
  };
  // the item's Q and dO rows are read from registers only by the score
  // products (the later products read the LDS tiles): once those are issued,
  // the next item's loads go into the same registers
  KeyItem<HD> it;
  auto compute = [&](int k) {
    const int i0 = 32 * nth_bit(qmask, k / gs);
    float Di = it.dws;
    if (a.O) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < HD; ++t) s = fmaf(it.o[t], it.fo[t], s);
      Di = s + __shfl_xor(s, 32);
    }
    if (hf == 0) {
      sL[l32] = it.lse * ATTN_LOG2E;
      sD[l32] = Di;
    }
    store_half<HD>(sQ + l32 * LDT + hf * HD, it.q);
    store_half<HD>(sO + l32 * LDT + hf * HD, it.o);
    // S = Q K^T and dP = dO V^T: register r <-> query crow(r, hf), lane <-> key
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int t = 0; t < HD; ++t) {
      s = mfma32(it.q[t], kB[t], s);
      dp = mfma32(it.o[t], vB[t], dp);
    }
    issue(k + 4, it);  // in flight during the rest of this item
    __builtin_amdgcn_wave_barrier();  // the item's rows and constants are in LDS
    // LSE, D and seg of this lane's rows crow(r, hf) = 8 (r / 4) + 4 hf + r % 4:
    // four consecutive rows per 16-byte read (a row past the end reads the
    // staged padding, seg = ~0: it sees nothing)
    float lse[16], dd[16];
    uint32_t sg[16];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int row0 = 8 * a4 + 4 * hf;
      const float4 l4 = *reinterpret_cast<const float4*>(sL + row0);
      const float4 d4 = *reinterpret_cast<const float4*>(sD + row0);
      const uint4 s4 = *reinterpret_cast<const uint4*>(sSeg + i0 + row0);
      lse[4 * a4] = l4.x; lse[4 * a4 + 1] = l4.y; lse[4 * a4 + 2] = l4.z; lse[4 * a4 + 3] = l4.w;
      dd[4 * a4] = d4.x; dd[4 * a4 + 1] = d4.y; dd[4 * a4 + 2] = d4.z; dd[4 * a4 + 3] = d4.w;
      sg[4 * a4] = s4.x; sg[4 * a4 + 1] = s4.y; sg[4 * a4 + 2] = s4.z; sg[4 * a4 + 3] = s4.w;
    }
    // the B operands of the products below, read while the probabilities
    // are formed
    float ob[16][NC], qb[16][NC];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ro = crow(r, hf) * LDT + l32;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        ob[r][c] = sO[ro + 32 * c];
        qb[r][c] = sQ[ro + 32 * c];
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int iq = i0 + crow(r, hf);
      const bool vis = sg[r] <= (uint32_t)j && j <= iq;
      // computed unconditionally and then selected (no branch; a masked
      // entry's value, possibly inf, is discarded)
      const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse[r]));
      const float p = vis ? e : 0.f;
      s[r] = p;
      dp[r] = p * (dp[r] - dd[r]);  // dS / scale
    }
    // dV += P^T dO, dK += dS^T Q: A = registers (lane <-> key), B = the tiles
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        accV[c] = mfma32(s[r], ob[r][c], accV[c]);
        accK[c] = mfma32(dp[r], qb[r][c], accK[c]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  issue(wave, it);
  for (int k = wave; k < nitems; k += 4) compute(k);

  __syncthreads();  // the LDS is now the reduction buffer: [4][32][DP] for dK, then for dV
  float* sRK = lds;
  float* sRV = lds + 4 * 32 * DP;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = (wave * 32 + crow(r, hf)) * DP + 32 * c + l32;
      sRK[e] = accK[c][r];
      sRV[e] = accV[c][r];
    }
  __syncthreads();
  const size_t slice = (size_t)S * a.KV * d;
  float* pK = a.part + (size_t)(2 * split) * slice;
  float* pV = pK + slice;
#pragma unroll
  for (int n = 0; n < BlockOut<DP>::N; ++n) {
    const int e = tid + 256 * n, row = e / DP, col = e % DP;
    if (j0 + row < S && col < d) {
      const float tk = ((sRK[e] + sRK[32 * DP + e]) + sRK[64 * DP + e]) + sRK[96 * DP + e];
      const float tv = ((sRV[e] + sRV[32 * DP + e]) + sRV[64 * DP + e]) + sRV[96 * DP + e];
      const size_t o = ((size_t)(j0 + row) * a.KV + kvh) * d + col;
      if (a.ksplit == 1) {
        a.dK[o] = outK.old[n] + a.scale * tk;
        a.dV[o] = outV.old[n] + tv;
      } else {
        pK[o] = a.scale * tk;
        pV[o] = tv;
      }
    }
  }
}

// One launch of the backward: blocks [0, nqb*KV*ksplit) take the key role
// (key block ascending: the first ones see the most queries; its KV heads
// and head splits adjacent), the rest the query role (query block
// descending, likewise).  ROWTERM: the query role only, writing D.
template <int DP, bool ROWTERM>
__global__ __launch_bounds__(256) void k_short(ShortArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[ShortGeom<DP>::LDS_FLOATS];
  __shared__ __attribute__((aligned(16))) float sRow[4 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t sSeg[SHORT_MAX_S];
  const int b = blockIdx.x;
  const int nkey = ROWTERM ? 0 : a.nqb * a.KV * a.ksplit;
  if (b < nkey) {
    const int kvh = b % a.KV, r = b / a.KV;
    short_key<DP>(a, r / a.ksplit, kvh, r % a.ksplit, lds, sRow, sSeg);
  } else {
    const int q = b - nkey;
    short_query<DP, ROWTERM>(a, a.nqb - 1 - q / a.H, q % a.H, lds, sSeg);
  }
}

// dK += sum over splits of part[2 split], dV += sum of part[2 split + 1],
// split by split in order; n = S * KV * d floats per slice (a multiple of 4).
__global__ __launch_bounds__(256) void k_short_sum(const float* __restrict__ part, int splits,
                                                   long long n, float* dK, float* dV) {
  const long long n4 = n / 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    float4 k = reinterpret_cast<float4*>(dK)[i], v = reinterpret_cast<float4*>(dV)[i];
    for (int s = 0; s < splits; ++s) {
      const float4 pk = reinterpret_cast<const float4*>(part + (size_t)(2 * s) * n)[i];
      const float4 pv = reinterpret_cast<const float4*>(part + (size_t)(2 * s + 1) * n)[i];
      k.x += pk.x; k.y += pk.y; k.z += pk.z; k.w += pk.w;
      v.x += pv.x; v.y += pv.y; v.z += pv.z; v.w += pv.w;
    }
    reinterpret_cast<float4*>(dK)[i] = k;
    reinterpret_cast<float4*>(dV)[i] = v;
  }
}

template <int DP>
static attn_status_t launch_short(const ShortArgs& a, bool rowterm, hipStream_t st) {
  if (rowterm) {
    hipLaunchKernelGGL((k_short<DP, true>), dim3(a.nqb * a.H), dim3(256), 0, st, a);
    return hip_check(hipGetLastError(), "launching k_short (row term)");
  }
  hipLaunchKernelGGL((k_short<DP, false>), dim3(a.nqb * (a.KV * a.ksplit + a.H)), dim3(256), 0,
                     st, a);
  return hip_check(hipGetLastError(), "launching k_short");
}

extern "C" attn_status_t attn_bwd_short(const float* Q, const float* K, const float* V,
                                        const float* O, const float* dO, const float* LSE,
                                        const uint32_t* seg, float* dQ, float* dK, float* dV,
                                        int seq_len, int n_heads, int n_kv_heads, int head_dim,
                                        float scale, void* stream) {
  clear_error();
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len > SHORT_MAX_S)
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len = %d is above %d (use attn_bwd or attn_bwd_o)",
                seq_len, SHORT_MAX_S);
  // a wave keeps its rows' halves of K, V (key role) or Q, dO (query role)
  // and two items' operand rows in registers, and each wave stages two
  // 32-row tiles in LDS: above 128 columns neither fits (LDS alone would be
  // 4 * 2 * 32 * (192 + 4) * 4 bytes = 200 KB at 192 columns).  Those head
  // dims run the general path's kernels (the same sums; several launches and
  // a workspace)
  if (head_dim > 128)
    return O ? attn_bwd_o(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads,
                          head_dim, scale, stream)
             : attn_bwd(Q, K, V, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                        scale, stream);
  // the kernels address every tensor with 32-bit byte offsets
  if ((long long)seq_len * n_heads * head_dim * 4 >= (1LL << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len * n_heads * head_dim * 4 = %lld bytes is 2^31 or more",
                (long long)seq_len * n_heads * head_dim * 4);
  if (seq_len == 0) return ATTN_OK;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  ShortArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.LSE = LSE; a.seg = seg;
  a.dQ = dQ; a.dK = dK; a.dV = dV; a.Dws = nullptr; a.part = nullptr;
  a.S = seq_len; a.H = n_heads; a.KV = n_kv_heads; a.d = head_dim;
  a.nqb = (seq_len + 31) / 32;
  a.scale = scale;
  const int dp = head_dim <= 32 ? 32 : head_dim <= 64 ? 64 : head_dim <= 96 ? 96 : 128;
  auto launch = [&](bool rowterm) {
    switch (dp) {
      case 32: return launch_short<32>(a, rowterm, st);
      case 64: return launch_short<64>(a, rowterm, st);
      case 96: return launch_short<96>(a, rowterm, st);
      default: return launch_short<128>(a, rowterm, st);
    }
  };
  // head splits of the key role: the first key block of a long document
  // sees up to nqb query blocks times g heads, nqb g / 4 items per wave.
  // Split its heads (a power of two dividing g) while that chain is longer
  // than 8 items and than a wave's share of all the items (about
  // nqb (nqb + 1) H of them over the chip's 1024 SIMDs): beyond that the
  // launch is bound by the total work, which the split does not reduce
  const int g = n_heads / n_kv_heads;
  const double share = (double)a.nqb * (a.nqb + 1) * n_heads / 1024.0;
  int ksplit = 1;
  while (ksplit < g && g % (2 * ksplit) == 0 &&
         (double)a.nqb * g / (4.0 * ksplit) > std::max(8.0, share))
    ksplit *= 2;
  a.ksplit = ksplit;

  void* ws = nullptr;
  const size_t d_bytes = O ? 0 : ((size_t)seq_len * n_heads * 4 + 255) / 256 * 256;
  const size_t part_bytes = ksplit > 1 ? (size_t)2 * ksplit * seq_len * n_kv_heads * head_dim * 4 : 0;
  if (d_bytes + part_bytes > 0) {
    hipMemPool_t pool;
    rc = device_pool(&pool);
    if (rc != ATTN_OK) return rc;
    rc = hip_check(hipMallocFromPoolAsync(&ws, d_bytes + part_bytes, pool, st),
                   "hipMallocFromPoolAsync(workspace)");
    if (rc != ATTN_OK) return rc;
    if (!O) a.Dws = static_cast<float*>(ws);
    if (ksplit > 1) a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + d_bytes);
  }
  rc = profile_mark(st, true);
  if (rc == ATTN_OK && !O) {
    rc = launch(true);
    if (rc == ATTN_OK) rc = profile_mark(st);
  }
  if (rc == ATTN_OK) rc = launch(false);
  if (rc == ATTN_OK && ksplit > 1) {
    const long long n = (long long)seq_len * n_kv_heads * head_dim;
    const int blocks = (int)std::min<long long>((n / 4 + 255) / 256, 2048);
    hipLaunchKernelGGL(k_short_sum, dim3(blocks), dim3(256), 0, st, a.part, ksplit, n, dK, dV);
    rc = hip_check(hipGetLastError(), "launching k_short_sum");
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (ws) {
    attn_status_t rc2 = hip_check(hipFreeAsync(ws, st), "hipFreeAsync(workspace)");
    if (rc == ATTN_OK) rc = rc2;
  }
  return rc;
}
