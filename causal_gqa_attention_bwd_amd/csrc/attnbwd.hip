// attnbwd.hip -- causal grouped-query attention backward with a per-query
// document-start mask, for CDNA4 (gfx950 / MI355X), fp32 in and out, fp32
// matrix-core (MFMA) arithmetic.
//
// Operation: page "llm.istanbul -- 10_backward_attention.wgsl", header
// comment and kernel attention_backward (Pass A: P, dP, D and dV; Pass B: dS,
// dQ and dK; Final: owned += of dQ).  The page's design (one workgroup per
// (query, head), CAS-atomic dK/dV scatter) was made for WebGPU on Apple GPUs;
// here the same sums are re-tiled for 64-wide wavefronts and MFMA.
//
// Default path (the probability tiles fit the scratch budget), per call:
//   k_prep    per 32-row query block: seg min/max and scratch slot offsets.
//   k_dq      query-major, one workgroup per (query tile, head): S and dP
//             (2 MFMA contractions per visible pair), P, P*dP and
//             D = sum_j P*dP; stores the P and P*dP tiles.
//   k_dkdv_p  key-major, one workgroup per (key tile, KV head): owns its
//             dK/dV rows and sums the GQA group inside the workgroup (the
//             key-major, atomic-free idea of the page's
//             attention_backward_short_dKdV kernel); reads the tiles, forms
//             dS, runs P^T.dO and dS^T.Q (2 contractions), leaves dS.
//   k_dqs     query-major: dQ += dS.K from the dS tiles (1 contraction).
// Recompute path (over budget): k_dq accumulates A = sum_j P*dP*k_j and
//   B = sum_j P*k_j, so dQ = scale*(A - D*B) (4 contractions), then k_dkdv
//   recomputes S and dP per pair (4 contractions).
// attn_bwd_o: k_rowdot first computes D = dO.O from the forward output; the
//   same kernels then run in their D-known mode (dS formed by k_dq).
// k_fwd       the forward producing LSE (and optionally O) for the backward's
//             input, in one sweep with a running max (page "tang 0.2.0 --
//             src/gpu/llm.rs", causal_attention_fused; plus the document mask
//             and the LSE output).
//
// MFMA v_mfma_f32_32x32x2_f32 (C[32x32] += A[32x2] * B[2x32]) lane layout,
// checked on the device: lane l supplies A[l%32][l/32] and B[l/32][l%32]; it
// holds C[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator register r.  The
// contraction index of a product is free to permute as long as A and B agree,
// so for the d-contractions half-wave hf takes columns [hf*TH, hf*TH+TH) and
// lane reads are contiguous (ds_read_b128).  For the contractions over rows
// (keys or queries), register r of an accumulator tile is directly the A
// operand of the next product: no transposes anywhere.
//
// Masking selects the probability and score-gradient tiles (it never multiplies
// a score by zero), so an overflowing exp or a -inf LSE at an invisible
// position cannot leak into a visible row.  Input values themselves (K, V rows
// of a staged key tile; Q, dO rows of a staged query tile) still enter the
// tile products with a zero weight when invisible: finite inputs contribute
// exactly 0, non-finite ones would propagate.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <map>
#include <mutex>
#include <vector>

#include "common.h"

struct BwdArgs {
  const float *Q, *K, *V, *dO, *LSE;
  const uint32_t* seg;  // NULL = all zeros
  float *dQ, *dK, *dV;  // never overlap each other or an input
  float* Dws;            // [S, H] row term, written by k_dq, read by k_dkdv
  uint32_t* blk_min;     // [ceil(S/32)] min seg per 32-row query block (k_prep)
  uint32_t* blk_max;     // [ceil(S/32)] max seg per 32-row query block (k_prep)
  long long* slot_off;   // [ceil(S/32) + 1] first tile slot of each query block (k_prep)
  float* scratch;        // P and P*dP tiles of every visible pair, or NULL
  int S, H, KV, d;       // H, KV: the heads this launch covers (a chunk of KV groups, or
                         // a share of one group's heads; pointers start at its first)
  int Hs, KVs;           // row strides in heads: Q, dO, dQ, LSE, D rows hold Hs heads,
                         // K, V, dK, dV (and the partial dK, dV slices) rows KVs
  float scale;
  int pair;              // 1: block p serves tiles p and n-1-p (equal causal work)
  int rope;              // 1: rotate dQ, dK back by RoPE after the += (rope_bwd)
  int rope_old;          // k_dkdv_p with rope: 1 rotates dK's old contents with the sum (the
                         // first chunk to write these rows), 0 adds only the rotated sum
  int rope_pos;          // position of row 0 (the page's pos_offset)
  double rope_base;      // frequency base
  int hsplit;            // k_dkdv_p: blocks sharing one key tile's heads (1, or 2^k | g)
  float* part;           // [2 * (hsplit - 1)][S, KV, d] partial dK, dV of splits 1.., or NULL
};

struct FwdArgs {
  const float *Q, *K, *V;
  const uint32_t* seg;
  float *O, *LSE;
  int S, H, KV, d;
  float scale;
};

// Load the TH contraction columns [cb, cb+TH) of one row into registers
// (zero beyond head_dim or for an invalid row).
template <int TH>
__device__ __forceinline__ void load_row(const float* row, int cb, int d, bool ok, float* out) {
#pragma unroll
  for (int t = 0; t < TH; t += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok && cb + t < d) x = *reinterpret_cast<const float4*>(row + cb + t);
    out[t] = x.x; out[t + 1] = x.y; out[t + 2] = x.z; out[t + 3] = x.w;
  }
}

// Pin loop-invariant MFMA operands into accumulation registers (AGPRs): the
// matrix cores read A/B operands from AGPRs directly, and the architectural
// VGPRs stay free for keeping LDS reads in flight.
template <int N>
__device__ __forceinline__ void pin_agpr(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(v[i]));
}

// ---------------------------------------------------------------------------
// Streaming tiles into LDS.
//
// The backward kernels stage row tiles (K/V rows in k_dq, Q/dO rows in
// k_dkdv) with direct buffer->LDS loads (buffer_load_dwordx4 ... lds: each
// lane's 16 bytes land at the wave's LDS base + 16 * lane), double-buffered
// so the next tile streams in while the current one is multiplied.  A tile is
// kept row-major with rows padded to DP + 4 floats, so that the b128 reads of
// 32 rows at one column and the b32 reads of 32 columns of one row hit
// distinct banks, and every LDS address in the hot loops is one per-lane base
// plus a compile-time offset.  Each 1 KiB chunk of the padded tile is one
// wave-wide load.  Zero fill is left to the buffer range check: the buffer
// resource of a tile ends with the tile's last valid row, and lanes that land
// on a pad granule or past head_dim carry an offset beyond any range, so all
// of them deposit zeros without touching memory.
// ---------------------------------------------------------------------------
// Padded ROWS x DP tile filled by 1 KiB chunks.
template <int ROWS, int DP>
struct PadTile {
  static constexpr int LDR = DP + 4;                 // floats per padded row
  static constexpr int GPR = LDR / 4;                // 16-byte granules per padded row
  static constexpr int NCH = (ROWS * GPR + 63) / 64; // wave-wide loads per tile
  static constexpr int FLOATS = NCH * 256;           // LDS floats reserved (>= ROWS * LDR)
  static constexpr int CPW = (NCH + 3) / 4;          // loads per wave (some waves one fewer)
};

// Per-lane byte offsets, relative to a tile's first row, of the granules this
// lane loads for a padded ROWS x DP tile of a matrix whose rows are `stride`
// floats apart with d valid columns.  Computed once per kernel.
template <int ROWS, int DP>
struct TileLoader {
  using T = PadTile<ROWS, DP>;
  uint32_t off[T::CPW];

  __device__ __forceinline__ void init(size_t stride, int d, int wave_u, int lane) {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) {
      const int p = (wave_u + 4 * i) * 64 + lane;  // granule of the padded tile
      const int row = p / T::GPR, g4 = p % T::GPR;
      const bool ok = row < ROWS && g4 < DP / 4 && 4 * g4 < d;
      off[i] = ok ? (uint32_t)(((size_t)row * stride + 4 * g4) * 4) : ATTN_BUF_OOB;
    }
  }
  // Buffer resource of rows [r0, min(r0 + ROWS, S)) of the matrix starting at
  // `base` (already at the head's first column); no rows (live = false) gives
  // an empty range.
  __device__ __forceinline__ i32x4 rsrc(const float* base, int r0, int S, size_t stride, int d,
                                         bool live) const {
    const int rows = live ? min(S - r0, ROWS) : 0;
    const uint32_t nbytes = rows > 0 ? (uint32_t)(((size_t)(rows - 1) * stride + d) * 4) : 0u;
    return buf_rsrc(live ? base + (size_t)r0 * stride : base, nbytes);
  }
  // The i-th of this wave's loads of a tile into the padded LDS tile `lds`.
  __device__ __forceinline__ void load(int i, const i32x4& r, float* lds, int wave_u) const {
    const int chunk = wave_u + 4 * i;
    if (4 * (i + 1) <= T::NCH || chunk < T::NCH) dma16(r, off[i], lds + chunk * 256);
  }
  __device__ __forceinline__ void load_all(const i32x4& r, float* lds, int wave_u) const {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) load(i, r, lds, wave_u);
  }
  // The same with the tile given by its LDS byte address.
  __device__ __forceinline__ void load(int i, const i32x4& r, uint32_t lds_byte, int wave_u) const {
    const int chunk = wave_u + 4 * i;
    if (4 * (i + 1) <= T::NCH || chunk < T::NCH) dma16(r, off[i], lds_byte + chunk * 1024);
  }
  __device__ __forceinline__ void load_all(const i32x4& r, uint32_t lds_byte, int wave_u) const {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) load(i, r, lds_byte, wave_u);
  }
};

// Above 128 columns a pair of waves shares one 32x32 score block by role:
// role 0 forms the Q.K product, role 1 the dO.V product, over all DP columns,
// and they swap results through LDS; each then owns DP/2 output columns.
template <int DP>
struct Pair {
  static constexpr bool ROLE = DP > 128;
  static constexpr int DW = ROLE ? DP / 2 : DP;  // output columns owned by a wave
  static constexpr int NB = DW / 32;             // 32-column output blocks per wave
  static constexpr int TH = DP / 2;              // score contraction steps per half-wave
  static_assert(DW % 32 == 0, "whole 32-column blocks");
};

// Swap the role products of a wave pair through LDS (16 floats per lane).
__device__ __forceinline__ f32x16 pair_swap(float* sX, int wave, int lane, const f32x16& mine) {
  float* w = sX + (wave * 16) * 64 + lane;
#pragma unroll
  for (int r = 0; r < 16; ++r) w[r * 64] = mine[r];
  lds_barrier();
  const float* o = sX + ((wave ^ 1) * 16) * 64 + lane;
  f32x16 other;
#pragma unroll
  for (int r = 0; r < 16; ++r) other[r] = o[r * 64];
  return other;
}

// No side work inside a score loop.
struct NoSide {
  __device__ __forceinline__ void operator()(int) const {}
};

// 32x32 score block over DP columns: acc = A_lds[row a_row][:] . B_reg, where
// half-wave hf contracts columns [hf*TH, hf*TH + TH).  Two accumulation
// chains, summed at the end.  side(step) is called once per 4-column step
// (TH/4 steps) so that other instructions issue between the products.
template <int DP, class Side>
__device__ __forceinline__ f32x16 score_block(const float* tile, int a_row, int hf, const float* breg,
                                              const Side& side) {
  constexpr int TH = Pair<DP>::TH, LDR = DP + 4;
  const float* ap = tile + a_row * LDR + hf * TH;
  f32x16 c0 = zero16(), c1 = zero16();
#pragma unroll
  for (int t = 0; t < TH; t += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(ap + t);
    c0 = mfma32(a4.x, breg[t], c0);
    c1 = mfma32(a4.y, breg[t + 1], c1);
    side(t / 4);
    c0 = mfma32(a4.z, breg[t + 2], c0);
    c1 = mfma32(a4.w, breg[t + 3], c1);
  }
  return c0 + c1;
}

// Two independent 32x32 score blocks sharing the LDS row (S and dP of one block).
template <int DP, class Side>
__device__ __forceinline__ void score_pair(const float* tA, const float* tB, int a_row, int hf,
                                           const float* rA, const float* rB, f32x16& x, f32x16& y,
                                           const Side& side) {
  constexpr int TH = Pair<DP>::TH, LDR = DP + 4;
  const int o0 = a_row * LDR + hf * TH;
  f32x16 cx = zero16(), cy = zero16();
#pragma unroll
  for (int t = 0; t < TH; t += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(tA + o0 + t);
    const float4 b4 = *reinterpret_cast<const float4*>(tB + o0 + t);
    cx = mfma32(a4.x, rA[t], cx);
    cy = mfma32(b4.x, rB[t], cy);
    cx = mfma32(a4.y, rA[t + 1], cx);
    cy = mfma32(b4.y, rB[t + 1], cy);
    side(t / 4);
    cx = mfma32(a4.z, rA[t + 2], cx);
    cy = mfma32(b4.z, rB[t + 2], cy);
    cx = mfma32(a4.w, rA[t + 3], cx);
    cy = mfma32(b4.w, rB[t + 3], cy);
  }
  x = cx;
  y = cy;
}

// Spreads N loads over the STEPS steps of a score loop: step t issues loads
// [t*N/STEPS, (t+1)*N/STEPS).
template <int N, int STEPS, class Issue>
struct SpreadLoads {
  const Issue& issue;
  __device__ __forceinline__ void operator()(int t) const {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (j * STEPS >= t * N && j * STEPS < (t + 1) * N) issue(j);
  }
};

// Pair partners of a lane's NB values in the permuted column layout
// (value nb of lane l sits in column c0 + NB*(l%32) + nb, c0 even): the other
// column of a pair is in the same lane or, for odd NB, in lane l +- 1.
template <int NB>
__device__ __forceinline__ void rope_partners_perm(const float (&v)[NB], int l32, float (&pv)[NB]) {
  if constexpr (NB % 2 == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pv[nb] = v[nb ^ 1];
  } else if constexpr (NB == 1) {
    pv[0] = __shfl_xor(v[0], 1);
  } else {
    static_assert(NB == 3, "odd column counts per lane are 1 or 3");
    const float up = __shfl_down(v[0], 1);  // lane + 1, first column
    const float dn = __shfl_up(v[2], 1);    // lane - 1, last column
    if ((l32 & 1) == 0) { pv[0] = v[1]; pv[1] = v[0]; pv[2] = up; }
    else { pv[0] = dn; pv[1] = v[2]; pv[2] = v[1]; }
  }
}

// ---------------------------------------------------------------------------
// k_prep: per 32-row query block, the smallest and largest document start,
// and the slot offsets of the P / P*dP tile scratch.  A query block qb can see
// keys only in key blocks [blk_min/32, qb]; each (query block, key block)
// pair in that range owns one slot, numbered query block by query block.
// One workgroup; a block-wide scan per 1024 query blocks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_prep(const uint32_t* seg, int S, uint32_t* blk_min,
                                               uint32_t* blk_max, long long* slot_off) {
  __shared__ long long sScan[1024];
  const int nblk = (S + 31) / 32;
  const int t = threadIdx.x;
  long long carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    const int b = b0 + t;
    long long cnt = 0;
    if (b < nblk) {
      uint32_t mn = 0xffffffffu, mx = 0u;
      const int r1 = min(b * 32 + 32, S);
      for (int r = b * 32; r < r1; ++r) {
        const uint32_t v = seg ? seg[r] : 0u;
        mn = min(mn, v);
        mx = max(mx, v);
      }
      blk_min[b] = mn;
      blk_max[b] = mx;
      cnt = max(0ll, (long long)b - (long long)(mn / 32) + 1);
    }
    sScan[t] = cnt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
      const long long v = t >= o ? sScan[t - o] : 0;
      __syncthreads();
      sScan[t] += v;
      __syncthreads();
    }
    if (b < nblk) slot_off[b] = carry + sScan[t] - cnt;
    carry += sScan[1023];
    __syncthreads();
  }
  if (t == 0) slot_off[nblk] = carry;
}

// ---------------------------------------------------------------------------
// k_sumparts: dK += sum over splits of part[2 split], dV += sum of
// part[2 split + 1], split by split in order, over `rows` rows of `width`
// floats (a multiple of 4: d is a multiple of 16) that sit `stride` floats
// apart in dK, dV and each slice (a slice is rows * stride floats).  Adds the
// partial sums of the key-major passes that split a group's heads over
// workgroups; with a chunk of KV heads, dK, dV and part start at its first.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sumparts(const float* __restrict__ part, int splits,
                                                  long long rows, int width, long long stride,
                                                  float* dK, float* dV, int rope, int d,
                                                  int rope_pos, double rope_base) {
  const size_t slice = (size_t)rows * stride;
  // tpr threads (a power of two, at most 256) per row, 256 / tpr rows per block
  const int w4 = width / 4;
  int tpr = 1;
  while (tpr < w4 && tpr < 256) tpr <<= 1;
  const int rpb = 256 / tpr;
  for (long long r = (long long)blockIdx.x * rpb + threadIdx.x / tpr; r < rows;
       r += (long long)gridDim.x * rpb) {
    for (int c4 = threadIdx.x % tpr; c4 < w4; c4 += tpr) {
      const size_t off = (size_t)r * stride + 4 * c4;
      float4 k = *reinterpret_cast<float4*>(dK + off), v = *reinterpret_cast<float4*>(dV + off);
      for (int s = 0; s < splits; ++s) {
        const float4 pk = *reinterpret_cast<const float4*>(part + (size_t)(2 * s) * slice + off);
        const float4 pv = *reinterpret_cast<const float4*>(part + (size_t)(2 * s + 1) * slice + off);
        k.x += pk.x; k.y += pk.y; k.z += pk.z; k.w += pk.w;
        v.x += pv.x; v.y += pv.y; v.z += pv.z; v.w += pv.w;
      }
      if (rope) {  // dK = R^T (dK + sum of the parts): the float4 holds two pairs
        const int col = (4 * c4) % d;
        const long long pos = r + rope_pos;
        const double f0 = rope_freq(col, d, rope_base), f1 = rope_freq(col + 2, d, rope_base);
        const float x0 = rope_back(k.x, k.y, col, pos, f0), y0 = rope_back(k.y, k.x, col + 1, pos, f0);
        const float x1 = rope_back(k.z, k.w, col + 2, pos, f1);
        const float y1 = rope_back(k.w, k.z, col + 3, pos, f1);
        k.x = x0; k.y = y0; k.z = x1; k.w = y1;
      }
      *reinterpret_cast<float4*>(dK + off) = k;
      *reinterpret_cast<float4*>(dV + off) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// k_rowdot: the row term read off the forward output, D[s, h] = dO[s, h, :] .
// O[s, h, :] (rows s*H + h of the [S, H, d] tensors).  A group of TPR lanes
// (a power of two covering the row's d/4 float4s) takes one row; a wave takes
// 64/TPR rows per step of a grid-stride loop whose trip count is the same for
// every lane of a wave (the group sums are shuffles).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rowdot(const float* __restrict__ O,
                                                const float* __restrict__ dO, float* D,
                                                long long rows, int d) {
  const int lane = threadIdx.x & 63;
  const int nf4 = d / 4;
  int tpr = 1;
  while (tpr < nf4) tpr <<= 1;
  const int rpw = 64 / tpr, sub = lane / tpr, part = lane % tpr;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const long long nwaves = (long long)gridDim.x * (blockDim.x / 64);
  for (long long r0 = wave * rpw; r0 < rows; r0 += nwaves * rpw) {
    const long long row = r0 + sub;
    float acc = 0.f;
    if (row < rows && part < nf4) {
      const float4 x = reinterpret_cast<const float4*>(O + row * d)[part];
      const float4 y = reinterpret_cast<const float4*>(dO + row * d)[part];
      acc = x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    for (int o = tpr / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (row < rows && part == 0) D[row] = acc;
  }
}

// The P / P*dP scratch holds, per slot and head, two 32x32 tiles (P, then
// P*dP) of one (query block, key block) pair, stored in the register layout
// of the key-major kernel: element R*64 + L is what its lane L holds in
// register R, i.e. P[query crow(R, L/32)][key L%32].  Masked pairs are zero.
#define ATTN_TILE_FLOATS 2048

// ---------------------------------------------------------------------------
// k_dq: the query-major pass, one workgroup per (query tile of BR rows, head).
// Wave w owns query block qb (32 queries); with the role split (DP > 128) two
// waves share a block.  The key sweep streams 32-row K/V tiles through LDS:
// one barrier per tile, and the next tile's loads are issued once this tile's
// score products are under way.
//   ACC = true:  D and dQ (A, B accumulated as above, dQ = scale*(A - D*B)).
//   ACC = false: D, and the P and P*dP tiles of every visible pair stored for
//                the key-major kernel (which then forms dS; k_dqs adds dS*K).
//   DK = true:   D is given (in a.Dws, from the forward output), so dS/scale =
//                P*(dP - D) is formed here: ACC accumulates dQ = scale*sum dS K
//                alone (3 contractions), !ACC stores dS/scale in place of P*dP.
// ---------------------------------------------------------------------------
template <int DP, bool ACC, bool DK>
__global__ __launch_bounds__(256) void k_dq(BwdArgs a) {
  using PG = Pair<DP>;
  constexpr int QB = PG::ROLE ? 2 : 4, BR = 32 * QB, BC = 32;
  constexpr int LDR = DP + 4;
  constexpr int TILE = PadTile<BC, DP>::FLOATS;
  __shared__ __attribute__((aligned(1024))) float sKV[2][2 * TILE];
  __shared__ __attribute__((aligned(16))) float sX[PG::ROLE ? 4 * 16 * 64 : 4];
  __shared__ float sD[4 * 32];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int role = PG::ROLE ? (wave & 1) : 0;
  const int qb = PG::ROLE ? (wave >> 1) : wave;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int qt_hi = (S - 1) / BR;
  auto tile = [&](const int qt) __attribute__((always_inline)) {
  const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
  const int i0 = qt * BR;
  const int q = i0 + qb * 32 + l32;
  const bool q_ok = q < S;
  const size_t qstride = (size_t)a.Hs * d, kstride = (size_t)a.KVs * d;
  const float sc2 = a.scale * ATTN_LOG2E;
  const float* Kh = a.K + (size_t)kvh * d;
  const float* Vh = a.V + (size_t)kvh * d;

  // B operands of the score blocks: this lane's query row, half-wave hf's columns
  float qr[PG::TH], gr[PG::ROLE ? 1 : PG::TH];
  if constexpr (PG::ROLE) {
    load_row<PG::TH>((role ? a.dO : a.Q) + (size_t)q * qstride + (size_t)h * d, hf * PG::TH, d,
                     q_ok, qr);
  } else {
    load_row<PG::TH>(a.Q + (size_t)q * qstride + (size_t)h * d, hf * PG::TH, d, q_ok, qr);
    load_row<PG::TH>(a.dO + (size_t)q * qstride + (size_t)h * d, hf * PG::TH, d, q_ok, gr);
    pin_agpr<PG::TH>(gr);
  }
  pin_agpr<PG::TH>(qr);
  const float lse2 = q_ok ? a.LSE[(size_t)q * a.Hs + h] * ATTN_LOG2E : 0.f;
  const float Dk = (DK && q_ok) ? a.Dws[(size_t)q * a.Hs + h] : 0.f;  // given row term
  const uint32_t sq = (q_ok && a.seg) ? a.seg[q] : 0u;

  // smallest document start of the tile bounds the key sweep; the largest one
  // of the wave's block tells which key blocks the block sees entirely
  uint32_t mn = q_ok ? sq : 0xffffffffu, mx = q_ok ? sq : 0u;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) sMin[wave] = mn;
  __syncthreads();
  uint32_t tmin = sMin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tmin = min(tmin, sMin[w]);
  const int qblk = (i0 >> 5) + qb;
  const int q_first = i0 + qb * 32;
  // scratch slots of this wave's query block: key blocks [kb_lo, qblk]
  const bool store = !ACC && q_first < S;
  const int kb_lo = store ? (int)(a.blk_min[qblk] / 32) : 0;
  const long long slot0 = store ? a.slot_off[qblk] - kb_lo : 0;
  // lane's element offset in a stored tile (see ATTN_TILE_FLOATS)
  const int st_base = 64 * (4 * (l32 >> 3) + (l32 & 3)) + 32 * ((l32 >> 2) & 1) + 4 * hf;
  const bool rows_full = q_first + 31 < S;  // all 32 queries of the block exist

  const int last_q = min(i0 + BR, S) - 1;
  const int kt_lo = (int)(min(tmin, (uint32_t)last_q) / BC), kt_hi = last_q / BC;

  f32x16 accA[ACC ? PG::NB : 1], accB[ACC && !DK ? PG::NB : 1];
  if constexpr (ACC) {
#pragma unroll
    for (int nb = 0; nb < PG::NB; ++nb) {
      accA[nb] = zero16();
      if constexpr (!DK) accB[nb] = zero16();
    }
  }
  float Dp = 0.f;
  const int dcol0 = role * PG::DW;

  TileLoader<BC, DP> ld;
  ld.init(kstride, d, wave, lane);
  const uint32_t lds_kv = lds_addr(&sKV[0][0]);
  {
    const i32x4 rk = ld.rsrc(Kh, kt_lo * BC, S, kstride, d, true);
    const i32x4 rv = ld.rsrc(Vh, kt_lo * BC, S, kstride, d, true);
    ld.load_all(rk, lds_kv, wave);
    ld.load_all(rv, lds_kv + TILE * 4, wave);
  }
  constexpr int NLOAD = 2 * PadTile<BC, DP>::CPW;  // loads per wave per tile
  int buf = 0;
  // the previous tile's P and P.dP, stored after the barrier that follows
  // them: issued just before a barrier, the stores would hold it up until
  // memory acknowledged them (the barrier's wait counts stores too)
  bool pend = false;
  float* pend_at = nullptr;
  f32x16 pst, pdt;
  auto flush = [&]() {
    if (ACC || !pend) return;
    if (!PG::ROLE || role == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pend_at[8 * (r >> 2) + (r & 3)] = pst[r];
    }
    if (!PG::ROLE || role == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) pend_at[1024 + 8 * (r >> 2) + (r & 3)] = pdt[r];
    }
    pend = false;
  };
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    tile_barrier();  // tile kt resident; everyone done with tile kt-1
    if constexpr (PG::ROLE) flush();
    const float* sK = &sKV[buf][0];
    const float* sV = &sKV[buf][TILE];
    const uint32_t nxt = lds_kv + (buf ^ 1) * (2 * TILE * 4);
    const int j0 = kt * BC;
    // every key of the tile visible to every query of the block: no masking
    const bool full = rows_full && q_first >= j0 + 31 && mx <= (uint32_t)j0;

    // loads of the next tile into the other buffer (empty ranges after the
    // last tile), issued between the score products below
    const bool more = kt < kt_hi;
    const i32x4 rk = ld.rsrc(Kh, (kt + 1) * BC, S, kstride, d, more);
    const i32x4 rv = ld.rsrc(Vh, (kt + 1) * BC, S, kstride, d, more);
    auto issue = [&](int j) {
      if (j < NLOAD / 2) ld.load(j, rk, nxt, wave);
      else ld.load(j - NLOAD / 2, rv, nxt + TILE * 4, wave);
    };
    // Without roles the previous tile's stores (8 groups of four values) go
    // out first, then the loads, spread over the score products: stored all
    // at once after the barrier, they held up the first products (S=4096:
    // 1.32 -> 1.17 ms)
    auto issue2 = [&](int j) {
      if constexpr (!PG::ROLE && !ACC) {
        if (j < 8) {
          if (pend) {
            const f32x16& v = j < 4 ? pst : pdt;
            const int m = j & 3;
            *reinterpret_cast<float4*>(pend_at + (j < 4 ? 0 : 1024) + 8 * m) =
                make_float4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
          }
          return;
        }
        issue(j - 8);
      } else {
        issue(j);
      }
    };
    constexpr int NSP = (!PG::ROLE && !ACC) ? NLOAD + 8 : NLOAD;
    const SpreadLoads<NSP, PG::TH / 4, decltype(issue2)> spread{issue2};

    // B operands of the accumulation below (independent of the scores): read
    // them now so that the accumulation runs without LDS waits
    float kv[16][ACC ? PG::NB : 1];
    if constexpr (ACC) {
      const float* kb0 = sK + (4 * hf) * LDR + dcol0 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int nb = 0; nb < PG::NB; ++nb) kv[r][nb] = kb0[(8 * (r >> 2) + (r & 3)) * LDR + nb * 32];
    }

    // S^T = K Q^T and dP^T = V dO^T: 32 keys x this wave's 32 queries
    f32x16 st, dpt;
    if constexpr (PG::ROLE) {
      const f32x16 mine = score_block<DP>(role ? sV : sK, l32, hf, qr, spread);
      const f32x16 other = pair_swap(sX, wave, lane, mine);
      st = role ? other : mine;
      dpt = role ? mine : other;
    } else {
      score_pair<DP>(sK, sV, l32, hf, qr, gr, st, dpt, spread);
    }

    // P and P*dP (DK: P*(dP - D)) in place; this lane's query, key = j0 + crow(r, hf)
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[r], sc2, -lse2));
        const float pdp = p * (DK ? dpt[r] - Dk : dpt[r]);
        if constexpr (!DK) Dp += pdp;
        st[r] = p;
        dpt[r] = pdp;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + crow(r, hf);
        const bool vis = q_ok && key <= q && (uint32_t)key >= sq;
        const float e = __builtin_amdgcn_exp2f(fmaf(st[r], sc2, -lse2));
        const float p = vis ? e : 0.f;
        const float pdp = vis ? p * (DK ? dpt[r] - Dk : dpt[r]) : 0.f;
        if constexpr (!DK) Dp += pdp;
        st[r] = p;
        dpt[r] = pdp;
      }
    }
    // P and P.dP of a pair the key-major kernel will read: kept for storing,
    // transposed, right after the next barrier
    // (copied unconditionally, so that the previous values die at the flush)
    pend = !ACC && store && kt >= kb_lo && kt <= qblk;
    pend_at = pend ? a.scratch + ((slot0 + kt) * H + h) * ATTN_TILE_FLOATS + st_base : nullptr;
    pst = st;
    pdt = dpt;
    // A += (P.dP) K,  B += P K over the 32 keys (DK: A += (dS/scale) K only)
    if constexpr (ACC) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int nb = 0; nb < PG::NB; ++nb) {
          if constexpr (!DK) accB[nb] = mfma32(st[r], kv[r][nb], accB[nb]);
          accA[nb] = mfma32(dpt[r], kv[r][nb], accA[nb]);
        }
      }
    }
    buf ^= 1;
  }
  tile_barrier();  // the last (empty) loads have landed before the LDS is reused or released
  flush();

  // D of this lane's query: the two half-waves saw disjoint keys
  if constexpr (!DK) {
    const float Dq = Dp + __shfl_xor(Dp, 32);
    if (ACC && hf == 0) sD[wave * 32 + l32] = Dq;
    if (q_ok && hf == 0 && role == 0) a.Dws[(size_t)q * a.Hs + h] = Dq;
  }
  if constexpr (ACC) {
    __syncthreads();
    // dQ += scale * (A - D B): all old values are read first, then all written
    float* __restrict__ dQh = a.dQ + (size_t)h * d;
    float old[PG::NB][16];
#pragma unroll
    for (int nb = 0; nb < PG::NB; ++nb) {
      const int col = dcol0 + nb * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + qb * 32 + crow(r, hf);
        old[nb][r] = (row < S && col < d) ? dQh[(size_t)row * qstride + col] : 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < PG::NB; ++nb) {
      const int col = dcol0 + nb * 32 + l32;
      const double fq = a.rope ? rope_freq(col, d, a.rope_base) : 0.0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = crow(r, hf);
        const int row = i0 + qb * 32 + m;
        float v;
        if constexpr (DK)
          v = old[nb][r] + a.scale * accA[nb][r];
        else
          v = old[nb][r] + a.scale * (accA[nb][r] - sD[wave * 32 + m] * accB[nb][r]);
        // dQ = R^T (dQ + sum dS K); the pair partner column sits in lane l ^ 1
        if (a.rope) v = rope_back(v, __shfl_xor(v, 1), col, (long long)row + a.rope_pos, fq);
        if (row < S && col < d) dQh[(size_t)row * qstride + col] = v;
      }
    }
  }
  };
  // longest rows first; paired: then the mirror tile
  const int first = qt_hi - (int)(blockIdx.x / H), second = mirror_tile(first, qt_hi + 1, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // the first tile is done with the LDS
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_dqw: k_dq's storing mode above 128 columns (DP = 192, 256), sized for two
// workgroups per CU.  Same work per (query tile of 64 rows, head): waves 2qb
// (role 0: S = K Q^T, Q in registers) and 2qb + 1 (role 1: dP = V dO^T) of
// query block qb.  The LDS holds a K/V key tile in two column chunks, each
// with the columns both half-waves contract at one time (half-wave hf takes
// columns hf*TH + t; chunk c holds t in [c*TH/2, (c+1)*TH/2)), double
// buffered: 68 KB.  Role 0 forms P and hands it to role 1 through LDS (8 KB,
// one direction); role 1 forms P*dP (with D given: dS/scale = P (dP - D)) and
// the row term one tile later, beside role 0's next products (S=16384,
// d=256: 4.02 -> 3.85 ms against a barrier between the exponentials and
// P*dP).  Role 0 stores the P tiles, role 1 the P*dP tiles, each spread over
// the next tile's first products.  Two workgroups per CU put two
// waves on each SIMD (one workgroup of four waves with the whole tile in LDS
// left one), so one wave's products run while the other exponentiates,
// exchanges or waits at a barrier.
// ---------------------------------------------------------------------------
template <int DP>
struct WideGeom {
  static constexpr int TH = DP / 2;        // contraction columns per half-wave
  static constexpr int CC = TH / 2;        // per half-wave per chunk
  static constexpr int DC = 2 * CC;        // columns of a chunk row (both halves)
  static constexpr int LDC = DC + 4;       // LDS pitch of a chunk row
  using T = PadTile<32, DC>;
  static constexpr int CT = T::FLOATS;     // floats of a staged 32-row chunk tile
};

// Per-lane global byte offsets of the granules this wave loads into one
// column chunk of a 32-row tile: LDS granule g of a row holds columns
// c*CC + 4g (half 0, g < CC/4) or TH + c*CC + 4(g - CC/4) (half 1); columns at
// or past d, the pad granule and rows past 32 read zeros (offset beyond the
// buffer).
template <int DP>
struct ChunkLoader {
  using W = WideGeom<DP>;
  using T = typename W::T;
  uint32_t off[2][T::CPW];
  __device__ __forceinline__ void init(size_t stride, int d, int wave, int lane) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < T::CPW; ++i) {
        const int p = (wave + 4 * i) * 64 + lane;
        const int row = p / T::GPR, g = p % T::GPR;
        const int col = g < W::CC / 4 ? c * W::CC + 4 * g : W::TH + c * W::CC + 4 * (g - W::CC / 4);
        const bool ok = row < 32 && g < W::DC / 4 && col < d;
        off[c][i] = ok ? (uint32_t)(((size_t)row * stride + col) * 4) : ATTN_BUF_OOB;
      }
  }
  __device__ __forceinline__ void load(int c, int i, const i32x4& r, uint32_t lds_byte,
                                       int wave) const {
    const int chunk = wave + 4 * i;
    if (4 * (i + 1) <= T::NCH || chunk < T::NCH) dma16(r, off[c][i], lds_byte + chunk * 1024);
  }
};

// Buffer resource of rows [r0, min(r0 + 32, S)) of a [S, stride] matrix
// starting at `base` (the head's first column); empty when !live.
__device__ __forceinline__ i32x4 rows32_rsrc(const float* base, int r0, int S, size_t stride,
                                             int d, bool live = true) {
  const int rows = live ? min(S - r0, 32) : 0;
  const uint32_t nbytes = rows > 0 ? (uint32_t)(((size_t)(rows - 1) * stride + d) * 4) : 0u;
  return buf_rsrc(live ? base + (size_t)r0 * stride : base, nbytes);
}

template <int DP, bool DK>
__global__ __launch_bounds__(256, 2) void k_dqw(BwdArgs a) {
  using W = WideGeom<DP>;
  constexpr int BR = 64, BC = 32, TH = W::TH, CC = W::CC, LDC = W::LDC, CT = W::CT;
  constexpr int CPW = W::T::CPW;
  __shared__ __attribute__((aligned(1024))) float sKV[2][2 * CT];  // stages of (K chunk, V chunk)
  __shared__ __attribute__((aligned(16))) float sX[2 * 16 * 64];   // P of each query block
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int role = wave & 1, qb = wave >> 1;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int qt_hi = (S - 1) / BR;
  ChunkLoader<DP> ld;
  ld.init((size_t)a.KVs * d, d, wave, lane);
  auto tile = [&](const int qt) __attribute__((always_inline)) {
  const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
  const int i0 = qt * BR;
  const int q = i0 + qb * 32 + l32;
  const bool q_ok = q < S;
  const size_t qstride = (size_t)a.Hs * d, kstride = (size_t)a.KVs * d;
  const float sc2 = a.scale * ATTN_LOG2E;
  const float* Kh = a.K + (size_t)kvh * d;
  const float* Vh = a.V + (size_t)kvh * d;

  // B operands: this lane's row of Q (role 0) or dO (role 1), half-wave hf's columns
  float qr[TH];
  load_row<TH>((role ? a.dO : a.Q) + (size_t)q * qstride + (size_t)h * d, hf * TH, d, q_ok, qr);
  pin_agpr<TH>(qr);
  const float lse2 = q_ok ? a.LSE[(size_t)q * a.Hs + h] * ATTN_LOG2E : 0.f;
  const float Dk = (DK && q_ok) ? a.Dws[(size_t)q * a.Hs + h] : 0.f;
  const uint32_t sq = (q_ok && a.seg) ? a.seg[q] : 0u;

  uint32_t mn = q_ok ? sq : 0xffffffffu, mx = q_ok ? sq : 0u;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) sMin[wave] = mn;
  __syncthreads();
  uint32_t tmin = sMin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tmin = min(tmin, sMin[w]);
  const int qblk = (i0 >> 5) + qb;
  const int q_first = i0 + qb * 32;
  const bool store = q_first < S;
  const int kb_lo = store ? (int)(a.blk_min[qblk] / 32) : 0;
  const long long slot0 = store ? a.slot_off[qblk] - kb_lo : 0;
  const int st_base = 64 * (4 * (l32 >> 3) + (l32 & 3)) + 32 * ((l32 >> 2) & 1) + 4 * hf;
  const bool rows_full = q_first + 31 < S;
  const int last_q = min(i0 + BR, S) - 1;
  const int kt_lo = (int)(min(tmin, (uint32_t)last_q) / BC), kt_hi = last_q / BC;
  float Dp = 0.f;

  const uint32_t lds_kv = lds_addr(&sKV[0][0]);
  {  // chunk 0 of the first key tile into buffer 0
    const i32x4 rk = rows32_rsrc(Kh, kt_lo * BC, S, kstride, d);
    const i32x4 rv = rows32_rsrc(Vh, kt_lo * BC, S, kstride, d);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      ld.load(0, i, rk, lds_kv, wave);
      ld.load(0, i, rv, lds_kv + CT * 4, wave);
    }
  }
  // Role 0 forms P of tile kt and hands it over in sX; role 1 forms P*dP of
  // tile kt one tile later, at the start of tile kt + 1 (it keeps dP^T of kt
  // in registers), so that its arithmetic runs beside role 0's products and
  // no barrier sits between the exponentials and P*dP.  sX has one slot per
  // query block: role 1 reads P of kt before the chunk-1 barrier of kt + 1,
  // and role 0 writes P of kt + 1 after it.  Each role's values of a tile
  // are stored during the next tile's chunk-0 products.
  bool pend = false;
  float* pend_at = nullptr;
  f32x16 pv;
  auto flush = [&]() {
    if (!pend) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) pend_at[role * 1024 + 8 * (r >> 2) + (r & 3)] = pv[r];
    pend = false;
  };
  float* xch = sX + (qb * 16) * 64 + lane;
  f32x16 xprev = zero16();  // role 1: dP^T of the previous tile
  int kprev = -1;           // the previous tile (-1: none)
  // role 1: P*dP (DK: P*(dP - D)) of tile kp from its P in sX and dP^T in xprev
  auto finish_pdp = [&](int kp) __attribute__((always_inline)) {
    const int jp = kp * BC;
    const bool fullp = rows_full && q_first >= jp + 31 && mx <= (uint32_t)jp;
    f32x16 y;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = jp + crow(r, hf);
      const bool vis = fullp || (q_ok && key <= q && (uint32_t)key >= sq);
      const float p = xch[r * 64];  // role 0 of this block wrote it
      const float pdp = vis ? p * (DK ? xprev[r] - Dk : xprev[r]) : 0.f;
      if constexpr (!DK) Dp += pdp;
      y[r] = pdp;
    }
    pend = store && kp >= kb_lo && kp <= qblk;
    pend_at = pend ? a.scratch + ((slot0 + kp) * H + h) * ATTN_TILE_FLOATS + st_base : nullptr;
    pv = y;
  };
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    // the two column chunks of key tile kt: stage 2 (kt - kt_lo) + c sits in
    // buffer c
    f32x16 c0 = zero16(), c1 = zero16();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      tile_barrier();  // chunk c resident; everyone done with the stage before
      // role 1, chunk 0: P*dP of the previous tile (its P is in sX now)
      if (c == 0 && role == 1 && kprev >= 0) finish_pdp(kprev);
      // the previous tile's stores (chunk 0, four groups of four values) and
      // the next stage's loads into the other buffer (none after the last),
      // spread over the products below
      const bool more = c == 0 || kt < kt_hi;
      const int nkt = c == 0 ? kt : kt + 1;
      const i32x4 rk = rows32_rsrc(Kh, nkt * BC, S, kstride, d, more);
      const i32x4 rv = rows32_rsrc(Vh, nkt * BC, S, kstride, d, more);
      const uint32_t nxt = lds_kv + (c ^ 1) * (2 * CT * 4);
      auto issue = [&](int j) {
        if (j < 4) {
          if (c == 0 && pend) {
            float* dst = pend_at + role * 1024 + 8 * j;
            *reinterpret_cast<float4*>(dst) = make_float4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
          }
        } else if (j < 4 + CPW) {
          ld.load(c ^ 1, j - 4, rk, nxt, wave);
        } else {
          ld.load(c ^ 1, j - 4 - CPW, rv, nxt + CT * 4, wave);
        }
      };
      const SpreadLoads<4 + 2 * CPW, CC / 4, decltype(issue)> spread{issue};
      // this chunk's contraction steps t = c CC + u, from the chunk row's
      // half-wave hf part
      const float* ap = &sKV[c][role * CT] + l32 * LDC + hf * CC;
#pragma unroll
      for (int u = 0; u < CC; u += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(ap + u);
        c0 = mfma32(a4.x, qr[c * CC + u], c0);
        c1 = mfma32(a4.y, qr[c * CC + u + 1], c1);
        spread(u / 4);
        c0 = mfma32(a4.z, qr[c * CC + u + 2], c0);
        c1 = mfma32(a4.w, qr[c * CC + u + 3], c1);
      }
      if (c == 0) pend = false;  // chunk 0 issued the stores
    }
    // the key tile is complete: role 0 holds S^T, role 1 dP^T (lane <-> query,
    // register r <-> key j0 + crow(r, hf))
    f32x16 x = c0 + c1;
    const int j0 = kt * BC;
    const bool full = rows_full && q_first >= j0 + 31 && mx <= (uint32_t)j0;
    if (role == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + crow(r, hf);
        const bool vis = full || (q_ok && key <= q && (uint32_t)key >= sq);
        const float e = __builtin_amdgcn_exp2f(fmaf(x[r], sc2, -lse2));
        x[r] = vis ? e : 0.f;
        xch[r * 64] = x[r];
      }
      pend = store && kt >= kb_lo && kt <= qblk;
      pend_at = pend ? a.scratch + ((slot0 + kt) * H + h) * ATTN_TILE_FLOATS + st_base : nullptr;
      pv = x;
    } else {
      xprev = x;
    }
    kprev = kt;
  }
  tile_barrier();  // the last (empty) loads have landed; P of the last tile is in sX
  flush();
  if (role == 1 && kprev >= 0) {
    finish_pdp(kprev);
    flush();
  }
  if constexpr (!DK) {
    const float Dq = Dp + __shfl_xor(Dp, 32);
    if (q_ok && hf == 0 && role == 1) a.Dws[(size_t)q * a.Hs + h] = Dq;
  }
  };
  // longest rows first; paired: then the mirror tile
  const int first = qt_hi - (int)(blockIdx.x / H), second = mirror_tile(first, qt_hi + 1, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // the first tile is done with the LDS
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_dkdv: dK and dV, one workgroup per (key tile of BC = 64 rows, KV head).
// Wave w: key block kb = w / 2 (32 keys), and either query block qs = w % 2
// of each 64-row query tile (DP <= 128) or role w % 2 of the one 32-row query
// block of a tile (DP > 128).  The K/V columns of the wave's keys stay in
// registers.  The sweep visits, for query tiles from the last one down to the
// tile holding the first key (so the workgroups resident on one XCD stream the
// same tiles together), each head of the group, skipping tiles none of whose
// queries can see these keys; Q/dO tiles are streamed through LDS with one
// barrier per tile.  Partial dK/dV of the two query blocks are summed through
// LDS at the end; each (key, KV head) row has a single writer.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void k_dkdv(BwdArgs a) {
  using PG = Pair<DP>;
  constexpr int KB = 2, QS = PG::ROLE ? 1 : 2, BC = 32 * KB, BR = 32 * QS;
  constexpr int LDR = DP + 4;
  constexpr int TILE = PadTile<BR, DP>::FLOATS;
  static_assert(QS == 1 || 4 * TILE >= KB * 2 * PG::NB * 16 * 64, "reduction buffer fits");
  __shared__ __attribute__((aligned(1024))) float sQG[2][2 * TILE];
  __shared__ __attribute__((aligned(16))) float sRow[2][4][64];  // LSE, D, seg, unused
  __shared__ __attribute__((aligned(16))) float sX[PG::ROLE ? 4 * 16 * 64 : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int kb = wave >> 1;
  const int qs = PG::ROLE ? 0 : (wave & 1);
  const int role = PG::ROLE ? (wave & 1) : 0;
  const int S = a.S, H = a.H, KV = a.KV, d = a.d;
  const int g = H / KV;
  const int kvh = blockIdx.x % KV;
  auto tile = [&](const int kt) __attribute__((always_inline)) {
  const int j0 = kt * BC;
  const int key = j0 + kb * 32 + l32;
  const bool key_ok = key < S;
  const size_t qstride = (size_t)a.Hs * d, kstride = (size_t)a.KVs * d;
  const float sc2 = a.scale * ATTN_LOG2E;

  // B operands of the score blocks: this lane's key row, half-wave hf's columns
  float kr[PG::TH], vr[PG::ROLE ? 1 : PG::TH];
  if constexpr (PG::ROLE) {
    load_row<PG::TH>((role ? a.V : a.K) + (size_t)key * kstride + (size_t)kvh * d, hf * PG::TH, d,
                     key_ok, kr);
  } else {
    load_row<PG::TH>(a.K + (size_t)key * kstride + (size_t)kvh * d, hf * PG::TH, d, key_ok, kr);
    load_row<PG::TH>(a.V + (size_t)key * kstride + (size_t)kvh * d, hf * PG::TH, d, key_ok, vr);
    pin_agpr<PG::TH>(vr);
  }
  pin_agpr<PG::TH>(kr);

  f32x16 accK[PG::NB], accV[PG::NB];
#pragma unroll
  for (int nb = 0; nb < PG::NB; ++nb) { accK[nb] = zero16(); accV[nb] = zero16(); }

  const int jlast = min(j0 + BC, S) - 1;
  const int nqt = (S + BR - 1) / BR, qt0 = j0 / BR;
  const int nblk = (S + 31) / 32;
  const int dcol0 = role * PG::DW;

  // query tile t can see a key of this tile unless every query's document
  // starts after the tile's last key
  auto visible_tile = [&](int t) {
    uint32_t mn = 0xffffffffu;
#pragma unroll
    for (int b = 0; b < QS; ++b) {
      const int bi = t * QS + b;
      if (bi < nblk) mn = min(mn, a.blk_min[bi]);
    }
    return mn <= (uint32_t)jlast;
  };
  auto prev_tile = [&](int t) {  // largest visible tile index <= t, or -1
    for (; t >= qt0; --t)
      if (visible_tile(t)) return t;
    return -1;
  };
  auto next_tile = [&](int t) {  // smallest visible tile index >= t, or -1
    for (; t < nqt; ++t)
      if (visible_tile(t)) return t;
    return -1;
  };
  // paired: the upper half of the key tiles sweeps the query tiles upwards
  // (the mirrors start at staggered times; upwards they read the same query
  // tile together, as the first tiles do downwards)
  const bool up = a.pair && 2 * kt > (S + BC - 1) / BC - 1;
  TileLoader<BR, DP> ld;
  ld.init(qstride, d, wave, lane);
  const uint32_t lds_qg = lds_addr(&sQG[0][0]);
  // per-row values of a tile, one wave-wide 4-byte load per wave: wave 0 LSE,
  // wave 1 D (rows H floats apart), wave 2 seg, wave 3 nothing (empty range
  // into a spare slot); lanes past the tile read nothing
  const uint32_t row_off = lane < BR ? (uint32_t)(lane * (wave == 2 ? 4 : 4 * a.Hs)) : ATTN_BUF_OOB;
  auto row_rsrc = [&](int t, int hh, bool live) {
    const int i0 = t * BR, h = kvh * g + hh;
    const int rows = live ? min(S - i0, BR) : 0;
    const void* base = a.LSE;
    uint32_t nbytes = 0;
    if (rows > 0) {
      if (wave == 0 || wave == 1) {
        base = (wave == 0 ? a.LSE : a.Dws) + (size_t)i0 * a.Hs + h;
        nbytes = (uint32_t)(((rows - 1) * (size_t)a.Hs + 1) * 4);
      } else if (wave == 2 && a.seg) {
        base = a.seg + i0;
        nbytes = (uint32_t)(rows * 4);
      }
    }
    return buf_rsrc(base, nbytes);
  };
  constexpr int NLOAD = 2 * PadTile<BR, DP>::CPW + 1;  // loads per wave per item
  auto next_item = [&](int t, int hx, int& nt, int& nh) {  // item after (t, hx), nt = -1 at the end
    nt = t;
    nh = hx + 1;
    if (nh == g) { nh = 0; nt = up ? next_tile(t + 1) : prev_tile(t - 1); }
  };

  int qt = up ? next_tile(qt0) : prev_tile(nqt - 1), hh = 0, buf = 0;
  int nqt_ = -1, nhh = 0;
  uint32_t bmax = 0;
  if (qt >= 0) {
    const i32x4 rq = ld.rsrc(a.Q + (size_t)(kvh * g) * d, qt * BR, S, qstride, d, true);
    const i32x4 rg = ld.rsrc(a.dO + (size_t)(kvh * g) * d, qt * BR, S, qstride, d, true);
    ld.load_all(rq, lds_qg, wave);
    ld.load_all(rg, lds_qg + TILE * 4, wave);
    dma4(row_rsrc(qt, 0, true), row_off, &sRow[0][wave][0]);
    next_item(qt, 0, nqt_, nhh);
    const int bi = qt * QS + qs;  // may not exist in a partial last tile
    bmax = bi < nblk ? a.blk_max[bi] : 0u;
  }
  while (qt >= 0) {
    tile_barrier();  // this item resident; everyone done with the previous one
    const float* sQ = &sQG[buf][0];
    const float* sG = &sQG[buf][TILE];
    const int i0 = qt * BR;
    const int q_first = i0 + qs * 32, k_first = j0 + kb * 32;
    // every query of the block sees every key of the wave: no masking
    const bool full = q_first + 31 < S && q_first >= k_first + 31 && bmax <= (uint32_t)k_first;

    // loads of the next item into the other buffer (empty ranges after the
    // last item), issued between the score products below
    const bool more = nqt_ >= 0;
    const int nh_ = kvh * g + (more ? nhh : 0);
    const i32x4 rq = ld.rsrc(a.Q + (size_t)nh_ * d, nqt_ * BR, S, qstride, d, more);
    const i32x4 rg = ld.rsrc(a.dO + (size_t)nh_ * d, nqt_ * BR, S, qstride, d, more);
    const i32x4 rr = row_rsrc(nqt_, nhh, more);
    const uint32_t nxt = lds_qg + (buf ^ 1) * (2 * TILE * 4);
    float* nrow = &sRow[buf ^ 1][wave][0];
    auto issue = [&](int j) {
      constexpr int C = PadTile<BR, DP>::CPW;
      if (j < C) ld.load(j, rq, nxt, wave);
      else if (j < 2 * C) ld.load(j - C, rg, nxt + TILE * 4, wave);
      else dma4(rr, row_off, nrow);
    };
    const SpreadLoads<NLOAD, PG::TH / 4, decltype(issue)> spread{issue};

    // dO operands of the dV accumulation below (independent of the scores)
    float gv[16][PG::NB];
    const int ob = (qs * 32 + 4 * hf) * LDR + dcol0 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int nb = 0; nb < PG::NB; ++nb) gv[r][nb] = sG[ob + (8 * (r >> 2) + (r & 3)) * LDR + nb * 32];

    // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys
    f32x16 s, dp;
    if constexpr (PG::ROLE) {
      const f32x16 mine = score_block<DP>(role ? sG : sQ, l32, hf, kr, spread);
      const f32x16 other = pair_swap(sX, wave, lane, mine);
      s = role ? other : mine;
      dp = role ? mine : other;
    } else {
      score_pair<DP>(sQ, sG, qs * 32 + l32, hf, kr, vr, s, dp, spread);
    }

    // look one item further ahead (scalar loads, complete under the products)
    int nnqt = -1, nnhh = 0;
    uint32_t nbmax = 0;
    if (more) {
      next_item(nqt_, nhh, nnqt, nnhh);
      const int bi = nqt_ * QS + qs;
      nbmax = bi < nblk ? a.blk_max[bi] : 0u;
    }

    // P and (dP - D) P in place (scale is applied to dK at the end);
    // register r = query qs*32 + crow(r, hf), lane = key
    const float* rowv = &sRow[buf][0][qs * 32 + 4 * hf];
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -rowv[o] * ATTN_LOG2E));
        dp[r] = p * (dp[r] - rowv[64 + o]);
        s[r] = p;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qs * 32 + crow(r, hf);
        const int qi = i0 + row;
        const int o = 8 * (r >> 2) + (r & 3);
        const float lse2 = rowv[o] * ATTN_LOG2E;
        const float Dv = rowv[64 + o];
        const uint32_t sg = __float_as_uint(rowv[128 + o]);
        const bool vis = key <= qi && sg <= (uint32_t)key && qi < S;
        const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse2));
        const float p = vis ? e : 0.f;
        const float dsv = vis ? p * (dp[r] - Dv) : 0.f;
        s[r] = p;
        dp[r] = dsv;
      }
    }
    // Q operands of the dK accumulation, read while the dV products run
    float qv[16][PG::NB];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int nb = 0; nb < PG::NB; ++nb) qv[r][nb] = sQ[ob + (8 * (r >> 2) + (r & 3)) * LDR + nb * 32];
    // dV += P^T dO, then dK += (dS/scale)^T Q over the 32 queries
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int nb = 0; nb < PG::NB; ++nb) accV[nb] = mfma32(s[r], gv[r][nb], accV[nb]);
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int nb = 0; nb < PG::NB; ++nb) accK[nb] = mfma32(dp[r], qv[r][nb], accK[nb]);
    qt = nqt_;
    hh = nhh;
    nqt_ = nnqt;
    nhh = nnhh;
    bmax = nbmax;
    buf ^= 1;
  }
  tile_barrier();  // the last (empty) loads have landed before the LDS is reused or released

  if constexpr (QS > 1) {
    float* red = &sQG[0][0] + kb * (2 * PG::NB * 16 * 64) + lane;
    if (qs == 1) {
#pragma unroll
      for (int nb = 0; nb < PG::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[((0 * PG::NB + nb) * 16 + r) * 64] = accK[nb][r];
          red[((1 * PG::NB + nb) * 16 + r) * 64] = accV[nb][r];
        }
    }
    __syncthreads();
    if (qs == 0) {
#pragma unroll
    for (int nb = 0; nb < PG::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accK[nb][r] += red[((0 * PG::NB + nb) * 16 + r) * 64];
        accV[nb][r] += red[((1 * PG::NB + nb) * 16 + r) * 64];
      }
    }
  }
  if (qs == 0) {  // the other query block's waves only contributed partial sums
  // dK += scale * accK, dV += accV: all old values are read first, then all written
  float* __restrict__ dKh = a.dK + (size_t)kvh * d;
  float* __restrict__ dVh = a.dV + (size_t)kvh * d;
  float oldK[PG::NB][16], oldV[PG::NB][16];
#pragma unroll
  for (int nb = 0; nb < PG::NB; ++nb) {
    const int col = dcol0 + nb * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = j0 + kb * 32 + crow(r, hf);
      const bool ok = row < S && col < d;
      const size_t off = (size_t)row * kstride + col;
      oldK[nb][r] = ok ? dKh[off] : 0.f;
      oldV[nb][r] = ok ? dVh[off] : 0.f;
    }
  }
#pragma unroll
  for (int nb = 0; nb < PG::NB; ++nb) {
    const int col = dcol0 + nb * 32 + l32;
    const double fq = a.rope ? rope_freq(col, d, a.rope_base) : 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = j0 + kb * 32 + crow(r, hf);
      float vk = oldK[nb][r] + a.scale * accK[nb][r];
      // dK = R^T (dK + sum dS^T Q); the pair partner column sits in lane l ^ 1
      if (a.rope) vk = rope_back(vk, __shfl_xor(vk, 1), col, (long long)row + a.rope_pos, fq);
      if (row < S && col < d) {
        const size_t off = (size_t)row * kstride + col;
        dKh[off] = vk;
        dVh[off] = oldV[nb][r] + accV[nb][r];
      }
    }
  }
  }  // qs == 0
  };
  // low key tiles (most queries) first; paired: then the mirror tile
  const int first = (int)(blockIdx.x / KV), second = mirror_tile(first, (S + BC - 1) / BC, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // the first tile is done with the LDS
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_dkdv_p: dK and dV from the stored P and P*dP tiles.
// Same decomposition and sweep as k_dkdv -- one workgroup per (key tile of
// 64 rows, KV head), wave w on key block kb = w / 2 -- but the score
// products are not recomputed: per (query block, key block, head) the wave
// loads the two stored tiles (prefetched one item ahead into registers),
// forms dS/scale = P*dP - P*D (written back over P*dP for k_dqs) and runs
// the two accumulations dV += P^T dO and dK += (dS/scale)^T Q.  With a given
// row term (DK) the second tile already holds dS/scale.  Above 128 columns
// the two waves of a key block split the output columns instead of the query
// rows.  With hsplit > 1, hsplit workgroups share a key tile, each taking
// g / hsplit heads of the group: the first adds its sums into dK, dV like an
// unsplit one, the others write theirs to their own slices of `part`
// (k_sumparts then adds them, split by split): under a document mask one key
// tile's work can exceed the per-CU share of the whole launch, and the split
// halves the longest workgroups.  With RoPE each part is rotated back on its
// own (the rotation is linear).
//
// The sweep order (query tiles, then the heads of the split) lives in
// registers: the query tiles are scanned in segments of 64 (lane i <-> tile
// base -/+ i); a ballot gives the tiles any query of which sees these keys,
// and each lane keeps its tile's slot base for this wave's block pair.  The
// walk over a segment is scalar bit arithmetic, so no memory read sits
// between an item and the next one's prefetch.
//
// Output columns are permuted: lane l's accumulator block nb holds column
// dcol0 + NB*(l%32) + nb, so that the NB operands a lane needs per step are
// adjacent in LDS (one wide read) and its NB results adjacent in memory.
// ---------------------------------------------------------------------------
template <int DP, bool DK>
__global__ __launch_bounds__(256) void k_dkdv_p(BwdArgs a) {
  constexpr bool DSPLIT = DP > 128;
  constexpr int KB = 2, QS = DSPLIT ? 1 : 2, BC = 32 * KB, BR = 32 * QS;
  constexpr int DW = DSPLIT ? DP / 2 : DP, NB = DW / 32;
  constexpr int LDR = DP + 4;
  constexpr int TILE = PadTile<BR, DP>::FLOATS;
  constexpr int CPW = PadTile<BR, DP>::CPW;
  static_assert(QS == 1 || 4 * TILE >= KB * 2 * NB * 16 * 64, "reduction buffer fits");
  __shared__ __attribute__((aligned(1024))) float sQG[2][2 * TILE];
  __shared__ __attribute__((aligned(16))) float sRow[2][4][64];  // D of a tile (slot 0)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int kb = wave >> 1;
  const int qs = DSPLIT ? 0 : (wave & 1);
  const int dcol0 = DSPLIT ? (wave & 1) * DW : 0;
  const int S = a.S, H = a.H, KV = a.KV, d = a.d;
  const int g = H / KV, gs = g / a.hsplit;  // heads of the group per split
  // block -> (tile, head split, KV head), KV head fastest
  const int kvh = blockIdx.x % KV;
  const int split = (int)(blockIdx.x / KV) % a.hsplit;
  const int nkt = (S + BC - 1) / BC;
  auto tile = [&](const int kt) __attribute__((always_inline)) {
  const int j0 = kt * BC;
  // paired: the upper half of the key tiles sweeps the query tiles upwards
  const bool up = a.pair && 2 * kt > nkt - 1;
  const int kblk = kt * KB + kb;  // this wave's key block
  const int head0 = kvh * g + split * gs;
  const size_t qstride = (size_t)a.Hs * d, kstride = (size_t)a.KVs * d;

  f32x16 accK[NB], accV[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { accK[nb] = zero16(); accV[nb] = zero16(); }

  const int jlast = min(j0 + BC, S) - 1;
  const int nblk = (S + 31) / 32;
  // query tiles that can see these keys: [qt_lo, qt_hi]
  const int qt_lo = j0 / BR, qt_hi = (S - 1) / BR;

  // segment of 64 tiles in sweep order, from base (lane i <-> tile base - i
  // downwards, base + i upwards): the mask of tiles with a visible pair, and
  // this lane's slot base of the wave's (query block, key block) pair (-1: no
  // visible key in the pair)
  int seg = up ? qt_lo : qt_hi, sbv = -1;
  uint64_t mask = 0;
  auto tile_of = [&](int base, int i) { return up ? base + i : base - i; };
  auto build = [&](int base) {
    const int t = tile_of(base, lane);
    bool vis = false;
    int sb = -1;
    if (t >= qt_lo && t <= qt_hi) {
      uint32_t mn = 0xffffffffu, mine = 0xffffffffu;
#pragma unroll
      for (int b = 0; b < QS; ++b) {
        const int bi = t * QS + b;
        const uint32_t v = bi < nblk ? a.blk_min[bi] : 0xffffffffu;
        mn = min(mn, v);
        if (b == qs) mine = v;
      }
      vis = mn <= (uint32_t)jlast;
      const int qb = t * QS + qs;
      const int lo = (int)(mine / 32);
      if (vis && qb < nblk && kblk <= qb && kblk >= lo)
        sb = (int)a.slot_off[qb] + (kblk - lo);
    }
    sbv = sb;
    mask = __ballot(vis);
  };
  // step (li, hh) to the next item of the sweep; false at its end
  auto advance = [&](int& li, int& hh) -> bool {
    if (++hh < gs) return true;
    hh = 0;
    uint64_t rest = li < 0 ? mask : (li >= 63 ? 0ull : mask & (~0ull << (li + 1)));
    while (rest == 0) {
      seg = tile_of(seg, 64);
      if (seg < qt_lo || seg > qt_hi) return false;
      build(seg);
      rest = mask;
    }
    li = __builtin_ctzll(rest);
    return true;
  };
  auto item_slot = [&](int li, int hh) -> int {
    const int sb = __builtin_amdgcn_readlane(sbv, li);
    return sb < 0 ? -1 : sb * H + head0 + hh;
  };

  TileLoader<BR, DP> ld;
  ld.init(qstride, d, wave, lane);
  const uint32_t row_off = lane < BR ? (uint32_t)(lane * 4 * a.Hs) : ATTN_BUF_OOB;
  auto row_rsrc = [&](int t, int hh, bool live) {  // D of the tile's rows (wave 0 only)
    const int i0 = t * BR;
    const int rows = (live && wave == 0) ? min(S - i0, BR) : 0;
    return buf_rsrc(rows > 0 ? a.Dws + (size_t)i0 * a.Hs + head0 + hh : a.Dws,
                    rows > 0 ? (uint32_t)(((rows - 1) * (size_t)a.Hs + 1) * 4) : 0u);
  };
  const uint32_t lds_qg = lds_addr(&sQG[0][0]), lds_row = lds_addr(&sRow[0][wave][0]);
  constexpr uint32_t QG_BYTES = 2 * TILE * 4, ROW_BYTES = 4 * 64 * 4;
  float pn[16], pdn[16];  // the next item's stored tiles
  auto fetch_tiles = [&](int slot) {
#pragma unroll
    for (int r = 0; r < 16; ++r) { pn[r] = 0.f; pdn[r] = 0.f; }
    if (slot >= 0) {
      const float* t = a.scratch + (size_t)slot * ATTN_TILE_FLOATS + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pn[r] = t[64 * r];
        pdn[r] = t[1024 + 64 * r];
      }
    }
  };

  build(seg);
  int li = -1, hh = gs - 1, buf = 0, cslot = -1;
  bool has = advance(li, hh);
  if (has) {
    const int t = tile_of(seg, li);
    const i32x4 rq = ld.rsrc(a.Q + (size_t)(head0 + hh) * d, t * BR, S, qstride, d, true);
    const i32x4 rg = ld.rsrc(a.dO + (size_t)(head0 + hh) * d, t * BR, S, qstride, d, true);
    ld.load_all(rq, lds_qg, wave);
    ld.load_all(rg, lds_qg + TILE * 4, wave);
    if constexpr (!DK) dma4(row_rsrc(t, hh, true), row_off, lds_row);
    cslot = item_slot(li, hh);
    fetch_tiles(cslot);
  }
  // this lane's operand offset in a Q/dO tile: query row qs*32 + 4*hf (+ the
  // step's row), columns dcol0 + NB*l32 ..
  const int ob = (qs * 32 + 4 * hf) * LDR + dcol0 + NB * l32;
  while (has) {
    tile_barrier();  // this item resident; everyone done with the previous one
    const float* sQ = &sQG[buf][0];
    const float* sG = &sQG[buf][TILE];
    float p[16], pd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) { p[r] = pn[r]; pd[r] = pdn[r]; }
    const bool vis = cslot >= 0;
    const float* Dv = &sRow[buf][0][qs * 32 + 4 * hf];

    // the next item: its stored tiles into registers, its Q/dO/D rows into
    // the other buffers (issued between the dV products below)
    const bool more = advance(li, hh);
    const int nt = more ? tile_of(seg, li) : 0;
    const int nslot = more ? item_slot(li, hh) : -1;
    fetch_tiles(nslot);
    const int nh = head0 + (more ? hh : 0);
    const i32x4 rq = ld.rsrc(a.Q + (size_t)nh * d, nt * BR, S, qstride, d, more);
    const i32x4 rg = ld.rsrc(a.dO + (size_t)nh * d, nt * BR, S, qstride, d, more);
    const i32x4 rr = row_rsrc(nt, more ? hh : 0, more);
    const uint32_t nxt = lds_qg + (buf ^ 1) * QG_BYTES;
    const uint32_t nrow = lds_row + (buf ^ 1) * ROW_BYTES;
    auto issue = [&](int j) {
      if (j < CPW) ld.load(j, rq, nxt, wave);
      else if (j < 2 * CPW) ld.load(j - CPW, rg, nxt + TILE * 4, wave);
      else if constexpr (!DK) dma4(rr, row_off, nrow);
    };
    constexpr int NLOAD = 2 * CPW + (DK ? 0 : 1);

    if (vis) {
      // dO operands of all 16 steps, then dS/scale = P*dP - P*D
      float gv[16][NB], qv[16][NB];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* row = sG + ob + (8 * (r >> 2) + (r & 3)) * LDR;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) gv[r][nb] = row[nb];
      }
      if constexpr (!DK) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pd[r] = fmaf(-p[r], Dv[8 * (r >> 2) + (r & 3)], pd[r]);
      }
      // dV += P^T dO; the Q operands of the dK products and the next item's
      // loads go out between these products
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) accV[nb] = mfma32(p[r], gv[r][nb], accV[nb]);
        const float* row = sQ + ob + (8 * (r >> 2) + (r & 3)) * LDR;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) qv[r][nb] = row[nb];
        SpreadLoads<NLOAD, 16, decltype(issue)>{issue}(r);
      }
      // dK += (dS/scale)^T Q.  dS/scale replaces P*dP in the scratch for
      // k_dqs (all waves read this item's tiles before the barrier above; one
      // writer per tile), stored between these products: stored before the
      // dV products they held up the phase's start (S=4096: k_dkdv_p 1.28 ->
      // 1.25 ms).  With a given row term (DK) the tile already holds dS/scale.
      const bool wr = !DK && (!DSPLIT || (wave & 1) == 0);
      float* const tds = a.scratch + (size_t)cslot * ATTN_TILE_FLOATS + 1024 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) accK[nb] = mfma32(pd[r], qv[r][nb], accK[nb]);
        if (wr) tds[64 * r] = pd[r];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NLOAD; ++j) issue(j);
    }
    // keep the accumulators in AGPRs across the loop (both paths above meet here)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      asm volatile("" : "+a"(accK[nb]));
      asm volatile("" : "+a"(accV[nb]));
    }
    cslot = nslot;
    has = more;
    buf ^= 1;
  }
  tile_barrier();  // the last loads have landed before the LDS is reused or released

  if constexpr (QS > 1) {
    float* red = &sQG[0][0] + kb * (2 * NB * 16 * 64) + lane;
    if (qs == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[((0 * NB + nb) * 16 + r) * 64] = accK[nb][r];
          red[((1 * NB + nb) * 16 + r) * 64] = accV[nb][r];
        }
    }
    __syncthreads();
    if (qs == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accK[nb][r] += red[((0 * NB + nb) * 16 + r) * 64];
        accV[nb][r] += red[((1 * NB + nb) * 16 + r) * 64];
      }
    }
  }
  // The write-back goes through buffers over this key tile's rows (from the
  // KV head's first column): rows past S and columns past head_dim get an
  // offset beyond the range, so their loads read zero and their stores are
  // dropped, with no divergent branch in the epilogue.
  const int col0 = dcol0 + NB * l32;
  const uint32_t tbytes = (uint32_t)(((size_t)(min(BC, S - j0) - 1) * kstride + d) * 4);
  uint32_t offs[16][NB];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = kb * 32 + crow(r, hf);  // row within the tile
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      offs[r][nb] = (j0 + rr < S && col0 + nb < d)
                        ? (uint32_t)(((size_t)rr * kstride + col0 + nb) * 4) : ATTN_BUF_OOB;
  }
  double fq[NB];  // RoPE frequency of each of this lane's columns
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) fq[nb] = a.rope ? rope_freq(col0 + nb, d, a.rope_base) : 0.0;
  if (qs == 0 && split > 0) {
  // splits after the first: the partial sums scale * accK (rotated back by
  // RoPE, which is linear) and accV into this split's slices of part;
  // k_sumparts adds them to what the first split wrote
  const size_t slice = (size_t)S * kstride, tile0 = (size_t)j0 * kstride + (size_t)kvh * d;
  const auto rK = out_rsrc(a.part + (size_t)(2 * split - 2) * slice + tile0, tbytes);
  const auto rV = out_rsrc(a.part + (size_t)(2 * split - 1) * slice + tile0, tbytes);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = j0 + kb * 32 + crow(r, hf);
    float vk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vk[nb] = a.scale * accK[nb][r];
    if (a.rope) {
      float pv[NB];
      rope_partners_perm<NB>(vk, l32, pv);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vk[nb] = rope_back(vk[nb], pv[nb], col0 + nb, (long long)row + a.rope_pos, fq[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      buf_st(rK, offs[r][nb], vk[nb]);
      buf_st(rV, offs[r][nb], accV[nb][r]);
    }
  }
  } else if (qs == 0) {  // one split, or the first of several  // the other query block's waves only contributed partial sums
  // dK += scale * accK, dV += accV: all old values are read first, then all written
  const size_t tile0 = (size_t)j0 * kstride + (size_t)kvh * d;
  const auto rK = out_rsrc(a.dK + tile0, tbytes);
  const auto rV = out_rsrc(a.dV + tile0, tbytes);
  float oldK[16][NB], oldV[16][NB];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      oldK[r][nb] = buf_ld(rK, offs[r][nb]);
      oldV[r][nb] = buf_ld(rV, offs[r][nb]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = j0 + kb * 32 + crow(r, hf);
    float vk[NB];
    // a later chunk of the same dK rows adds R^T (sum) to what an earlier
    // chunk left (already rotated); otherwise dK = R^T (dK + sum dS^T Q)
    const bool add_after = a.rope && !a.rope_old;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      vk[nb] = (add_after ? 0.f : oldK[r][nb]) + a.scale * accK[nb][r];
    if (a.rope) {
      float pv[NB];
      rope_partners_perm<NB>(vk, l32, pv);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vk[nb] = rope_back(vk[nb], pv[nb], col0 + nb, (long long)row + a.rope_pos, fq[nb]);
    }
    if (add_after) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vk[nb] += oldK[r][nb];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      buf_st(rK, offs[r][nb], vk[nb]);
      buf_st(rV, offs[r][nb], oldV[r][nb] + accV[nb][r]);
    }
  }
  }  // qs == 0
  };
  // Low key tiles (most queries) first, sweeping the query tiles downwards:
  // the blocks of one KV head start together, so they all read the same
  // query tile at the same time.  Paired, the mirror tile follows and is
  // swept upwards: of n key tiles, mirror n-1-k starts after the n-k query
  // tiles of tile k, at its own lowest query tile, so all blocks are then at
  // query tile t-1 at time t and their Q and dO reads share L2 again
  // (downwards they would spread over all tiles).  Unpaired (documents), a
  // block's tile lies inside one document and the blocks of a document
  // start together, so downwards is kept.
  const int first = (int)(blockIdx.x / KV) / a.hsplit, second = mirror_tile(first, nkt, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // the first tile is done with the LDS
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_dqs: dQ += scale * sum_j (dS/scale)_ij k_j from the dS tiles k_dkdv_p left
// in the scratch.  One workgroup per (query tile, head); wave w owns query
// block qb and a DW-column slice (DP <= 128: 4 blocks, all columns; DP > 128:
// 2 blocks x 2 column halves).  The sweep streams 64-key K tiles through LDS
// (one barrier per tile; 32 keys above 128 columns) and prefetches the
// wave's dS tiles of the next tile into registers.  dS is zero wherever the mask hides a key, and pairs
// outside the stored range are skipped, so no masking is needed here.
// Output columns are permuted as in k_dkdv_p (lane l, block nb: column
// dcol0 + NB*(l%32) + nb).
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256, 2) void k_dqs(BwdArgs a) {
  constexpr bool CSPLIT = DP > 128;
  constexpr int QB = CSPLIT ? 2 : 4, BR = 32 * QB, KB = CSPLIT ? 1 : 2, BC = 32 * KB;
  constexpr int DW = CSPLIT ? DP / 2 : DP, NB = DW / 32;
  constexpr int LDR = DP + 4;
  constexpr int TILE = PadTile<BC, DP>::FLOATS;
  constexpr int CPW = PadTile<BC, DP>::CPW;
  __shared__ __attribute__((aligned(1024))) float sK[2][TILE];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int qb = CSPLIT ? (wave >> 1) : wave;
  const int dcol0 = CSPLIT ? (wave & 1) * DW : 0;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int qt_hi = (S - 1) / BR;
  auto tile = [&](const int qt) __attribute__((always_inline)) {
  const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
  const int i0 = qt * BR;
  const int nblk = (S + 31) / 32;
  const int qblk = (i0 >> 5) + qb;
  const bool blk_ok = qblk < nblk;
  // stored pairs of this wave's query block: key blocks [lo, qblk]
  const int lo = blk_ok ? (int)(a.blk_min[qblk] / 32) : 0x7fffffff;
  const long long slot0 = blk_ok ? a.slot_off[qblk] - lo : 0;
  if (lane == 0) sMin[wave] = (blk_ok && lo <= qblk) ? (uint32_t)lo : 0x7fffffffu;
  __syncthreads();
  int kb_first = (int)sMin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) kb_first = min(kb_first, (int)sMin[w]);
  // key tiles holding a stored pair of some block of the tile (none: empty range)
  const int last_blk = (min(i0 + BR, S) - 1) / 32;
  const bool any = kb_first <= last_blk;
  const int kt_lo = any ? kb_first / KB : 1, kt_hi = any ? last_blk / KB : 0;
  const size_t kstride = (size_t)a.KVs * d;
  const float* Kh = a.K + (size_t)kvh * d;
  // lane's offset in a stored tile: dS[query l32][key crow(r, hf)] sits at
  // st_base + 8*(r/4) + r%4
  const int st_base = 64 * (4 * (l32 >> 3) + (l32 & 3)) + 32 * ((l32 >> 2) & 1) + 4 * hf;

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = zero16();

  float sn[KB][16];  // the next tile's dS values of this wave (zero when not stored)
  auto fetch = [&](int t) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int kb = t * KB + k;
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[k][r] = 0.f;
      if (blk_ok && kb >= lo && kb <= qblk) {
        const float* src = a.scratch + ((slot0 + kb) * H + h) * ATTN_TILE_FLOATS + 1024 + st_base;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 v = *reinterpret_cast<const float4*>(src + 8 * m);
          sn[k][4 * m] = v.x; sn[k][4 * m + 1] = v.y; sn[k][4 * m + 2] = v.z; sn[k][4 * m + 3] = v.w;
        }
      }
    }
  };

  TileLoader<BC, DP> ld;
  ld.init(kstride, d, wave, lane);
  const uint32_t lds_k = lds_addr(&sK[0][0]);
  if (kt_lo <= kt_hi) {
    ld.load_all(ld.rsrc(Kh, kt_lo * BC, S, kstride, d, true), lds_k, wave);
    fetch(kt_lo);
  }
  const int ob = (4 * hf) * LDR + dcol0 + NB * l32;
  int buf = 0;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    tile_barrier();  // tile kt resident; everyone done with tile kt-1
    const float* sKt = &sK[buf][0];
    float sv[KB][16];
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[k][r] = sn[k][r];
    const bool more = kt < kt_hi;
    if (more) fetch(kt + 1);
    const i32x4 rk = ld.rsrc(Kh, (kt + 1) * BC, S, kstride, d, more);
    const uint32_t nxt = lds_k + (buf ^ 1) * (TILE * 4);
    auto issue = [&](int j) { ld.load(j, rk, nxt, wave); };
    // (a block pair that holds no stored tile runs on zeros: no branches
    // here); step u = 16k + r, its K operands read one step ahead
    auto krow = [&](int u) { return sKt + ob + (32 * (u >> 4) + 8 * ((u >> 2) & 3) + (u & 3)) * LDR; };
    float kv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) kv[nb] = krow(0)[nb];
#pragma unroll
    for (int u = 0; u < 16 * KB; ++u) {
      float kn[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) kn[nb] = u + 1 < 16 * KB ? krow(u + 1)[nb] : kv[nb];
      __builtin_amdgcn_sched_barrier(0);  // keep the reads a full step ahead
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma32(sv[u >> 4][u & 15], kv[nb], acc[nb]);
      if (u < 16) SpreadLoads<CPW, 16, decltype(issue)>{issue}(u);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) kv[nb] = kn[nb];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+a"(acc[nb]));
    buf ^= 1;
  }
  tile_barrier();  // the last loads have landed before the LDS is released

  // dQ += scale * acc: all old values are read first, then all written
  float* __restrict__ dQh = a.dQ + (size_t)h * d;
  const size_t qstride = (size_t)a.Hs * d;
  const int col0 = dcol0 + NB * l32;
  float old[16][NB];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = i0 + qb * 32 + crow(r, hf);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      old[r][nb] = (row < S && col0 + nb < d) ? dQh[(size_t)row * qstride + col0 + nb] : 0.f;
  }
  double fq[NB];  // RoPE frequency of each of this lane's columns
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) fq[nb] = a.rope ? rope_freq(col0 + nb, d, a.rope_base) : 0.0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = i0 + qb * 32 + crow(r, hf);
    float v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) v[nb] = old[r][nb] + a.scale * acc[nb][r];
    if (a.rope) {  // dQ = R^T (dQ + sum dS K)
      float pv[NB];
      rope_partners_perm<NB>(v, l32, pv);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        v[nb] = rope_back(v[nb], pv[nb], col0 + nb, (long long)row + a.rope_pos, fq[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (row < S && col0 + nb < d) dQh[(size_t)row * qstride + col0 + nb] = v[nb];
  }
  };
  // longest rows first; paired: then the mirror tile
  const int first = qt_hi - (int)(blockIdx.x / H), second = mirror_tile(first, qt_hi + 1, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // the first tile is done with the LDS
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_fwd: the forward that produces the backward's inputs, LSE and (WANT_O) O,
// in one sweep with a running max (page "tang 0.2.0 -- src/gpu/llm.rs",
// causal_attention_fused: row max, exp-sum, probability-weighted V; here
// with the document mask, the log-sum-exp output, and the max carried across
// key tiles, O being rescaled when it moves).  One workgroup per (query tile
// of 128 rows, head); wave w owns query block w (32 queries) and all DP
// columns.  K/V tiles of 32 keys are streamed through LDS as in k_dq.
//   S^T = K Q^T  (lane <-> query, register r <-> key crow(r, hf)),
//   m' = max(m, max over the tile), alpha = 2^(m - m'), p = 2^(x - m'),
//   l = alpha*l + sum p,  O = alpha*O + P V   (log2 domain, x = scale*s*log2e).
// O's rows sit in register r (query crow(r, hf)), so each row's alpha and
// final 1/l come from the lane holding that query (a shuffle).  O's columns
// are permuted (lane l, block nb <-> column NB*(l%32) + nb) so a step's V
// operands are one wide LDS read.
// ---------------------------------------------------------------------------
template <int DP, bool WANT_O>
__global__ __launch_bounds__(256) void k_fwd(FwdArgs a) {
  constexpr int QB = 4, BR = 32 * QB, BC = 32;
  constexpr int LDR = DP + 4, TH = DP / 2, NB = DP / 32;
  constexpr int TILE = PadTile<BC, DP>::FLOATS;
  constexpr int CPW = PadTile<BC, DP>::CPW;
  __shared__ __attribute__((aligned(1024))) float sKV[2][2 * TILE];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int qt_hi = (S - 1) / BR;
  const int qt = qt_hi - (int)(blockIdx.x / H);  // longest rows first
  const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
  const int i0 = qt * BR;
  const int q = i0 + wave * 32 + l32;
  const bool q_ok = q < S;
  const size_t qstride = (size_t)H * d, kstride = (size_t)a.KV * d;
  const float sc2 = a.scale * ATTN_LOG2E;
  const float* Kh = a.K + (size_t)kvh * d;
  const float* Vh = a.V + (size_t)kvh * d;

  // B operand of the score block: this lane's query row, half-wave hf's columns
  float qr[TH];
  load_row<TH>(a.Q + (size_t)q * qstride + (size_t)h * d, hf * TH, d, q_ok, qr);
  pin_agpr<TH>(qr);
  const uint32_t sq = (q_ok && a.seg) ? a.seg[q] : 0u;
  uint32_t mn = q_ok ? sq : 0xffffffffu;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
  if (lane == 0) sMin[wave] = mn;
  __syncthreads();
  uint32_t tmin = sMin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tmin = min(tmin, sMin[w]);
  const int last_q = min(i0 + BR, S) - 1;
  const int kt_lo = (int)(min(tmin, (uint32_t)last_q) / BC), kt_hi = last_q / BC;

  float m = -INFINITY, l = 0.f;  // this lane's query: running max, this half's running sum
  f32x16 accO[WANT_O ? NB : 1];
  if constexpr (WANT_O) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) accO[nb] = zero16();
  }

  TileLoader<BC, DP> ld;
  ld.init(kstride, d, wave, lane);
  const uint32_t lds_kv = lds_addr(&sKV[0][0]);
  {
    ld.load_all(ld.rsrc(Kh, kt_lo * BC, S, kstride, d, true), lds_kv, wave);
    if constexpr (WANT_O) ld.load_all(ld.rsrc(Vh, kt_lo * BC, S, kstride, d, true), lds_kv + TILE * 4, wave);
  }
  constexpr int NLOAD = (WANT_O ? 2 : 1) * CPW;
  const int ob = (4 * hf) * LDR + NB * l32;  // this lane's V operands (row 4*hf + step row)
  int buf = 0;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    tile_barrier();  // tile kt resident; everyone done with tile kt-1
    const float* sK = &sKV[buf][0];
    const float* sV = &sKV[buf][TILE];
    const uint32_t nxt = lds_kv + (buf ^ 1) * (2 * TILE * 4);
    const int j0 = kt * BC;
    const bool more = kt < kt_hi;
    const i32x4 rk = ld.rsrc(Kh, (kt + 1) * BC, S, kstride, d, more);
    const i32x4 rv = ld.rsrc(Vh, (kt + 1) * BC, S, kstride, d, more && WANT_O);
    auto issue = [&](int j) {
      if (j < CPW) ld.load(j, rk, nxt, wave);
      else ld.load(j - CPW, rv, nxt + TILE * 4, wave);
    };
    const SpreadLoads<NLOAD, TH / 4, decltype(issue)> spread{issue};
    const f32x16 st = score_block<DP>(sK, l32, hf, qr, spread);

    // running max over this tile's visible keys (both half-waves hold the query)
    float x[16], mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + crow(r, hf);
      const bool vis = q_ok && key <= q && (uint32_t)key >= sq;
      x[r] = vis ? st[r] * sc2 : -INFINITY;
      mloc = fmaxf(mloc, x[r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(m, mloc);
    // alpha rescales what was summed under the old max (nothing yet: 0)
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
    float p[16], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = (x[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[r] - mnew);
      psum += p[r];
    }
    if (mnew != -INFINITY) {
      l = l * alpha + psum;
      m = mnew;
    }
    if constexpr (WANT_O) {
      // rescale O's rows when some query's max moved (alpha != 1)
      const bool moved = mnew != -INFINITY && alpha != 1.f;
      if (__ballot(moved)) {
        const float am = moved ? alpha : 1.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ar = __shfl(am, crow(r, hf));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) accO[nb][r] *= ar;
        }
      }
      // O += P V over the 32 keys
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* vrow = sV + ob + (8 * (r >> 2) + (r & 3)) * LDR;
        float vv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vv[nb] = vrow[nb];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) accO[nb] = mfma32(p[r], vv[nb], accO[nb]);
      }
    }
    buf ^= 1;
  }
  tile_barrier();  // the last (empty) loads have landed before the LDS is released

  // LSE = ln(sum) = (m + log2 L) * ln 2, L summed over both half-waves
  const float L = l + __shfl_xor(l, 32);
  const float lse2 = (m == -INFINITY || !(L > 0.f)) ? -INFINITY : m + log2f(L);
  if (q_ok && hf == 0) a.LSE[(size_t)q * H + h] = lse2 * ATTN_LN2;
  if constexpr (WANT_O) {
    const float inv = (lse2 == -INFINITY) ? 0.f : 1.f / L;
    float* __restrict__ Oh = a.O + (size_t)h * d;
    const int col0 = NB * l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float ir = __shfl(inv, crow(r, hf));
      const int row = i0 + wave * 32 + crow(r, hf);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (row < S && col0 + nb < d) Oh[(size_t)row * qstride + col0 + nb] = accO[nb][r] * ir;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static thread_local char g_err[512];

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = 0; }

extern "C" const char* attn_last_error(void) { return g_err; }

// Per-thread event log of the measurement hooks (see attn_profile_begin):
// per recorded attn_bwd call, one event before its first pass and one after
// each of its passes (2 or 3, or 3 per head chunk).
struct ProfileLog {
  bool on = false;
  std::vector<std::vector<hipEvent_t>> calls;
};
static thread_local ProfileLog g_prof;

static void profile_release() {
  for (auto& c : g_prof.calls)
    for (hipEvent_t e : c) (void)hipEventDestroy(e);
  g_prof.calls.clear();
}

extern "C" attn_status_t attn_profile_begin(void) {
  g_err[0] = 0;
  profile_release();
  g_prof.on = true;
  return ATTN_OK;
}

extern "C" attn_status_t attn_profile_end(double* ms, int* n_calls) {
  g_err[0] = 0;
  double sum[3] = {0.0, 0.0, 0.0};
  attn_status_t rc = ATTN_OK;
  for (size_t i = 0; i < g_prof.calls.size() && rc == ATTN_OK; ++i) {
    const auto& ev = g_prof.calls[i];
    // a call run in head chunks records its three passes once per chunk
    for (size_t k = 0; k + 1 < ev.size() && rc == ATTN_OK; ++k) {
      float t = 0.f;
      hipError_t e = hipEventSynchronize(ev[k + 1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[k], ev[k + 1]);
      if (e != hipSuccess) rc = fail(ATTN_ERR_HIP, "reading profile events: %s", hipGetErrorString(e));
      sum[k % 3] += t;
    }
  }
  if (ms) { ms[0] = sum[0]; ms[1] = sum[1]; ms[2] = sum[2]; }
  if (n_calls) *n_calls = (int)g_prof.calls.size();
  profile_release();
  g_prof.on = false;
  return rc;
}

// Record one profile event on `st` if the measurement hooks are on; `first`
// opens the record of a new call.
attn_status_t profile_mark(hipStream_t st, bool first) {
  if (!g_prof.on) return ATTN_OK;
  // timing only, so without the system-scope fence: its cache writeback and
  // invalidation would hold the stream a few microseconds between the passes
  // it measures
  hipEvent_t e;
  hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "profile event: %s", hipGetErrorString(err));
  err = hipEventRecord(e, st);
  if (err != hipSuccess) {
    (void)hipEventDestroy(e);
    return fail(ATTN_ERR_HIP, "profile event: %s", hipGetErrorString(err));
  }
  if (first || g_prof.calls.empty()) g_prof.calls.emplace_back();
  g_prof.calls.back().push_back(e);
  return ATTN_OK;
}

int padded_dim(int d) {
  if (d <= 32) return 32;
  if (d <= 64) return 64;
  if (d <= 96) return 96;
  if (d <= 128) return 128;
  if (d <= 192) return 192;
  return 256;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

attn_status_t check_common(int S, int H, int KV, int d, float scale) {
  if (S < 0) return fail(ATTN_ERR_INVALID_ARG, "seq_len = %d is negative", S);
  if (H < 1 || KV < 1) return fail(ATTN_ERR_INVALID_ARG, "n_heads = %d, n_kv_heads = %d", H, KV);
  if (H % KV != 0)
    return fail(ATTN_ERR_INVALID_ARG, "n_heads = %d is not a multiple of n_kv_heads = %d", H, KV);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
  if (d < 16 || d > 256 || d % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim = %d (supported: multiples of 16 in [16, 256])", d);
  if ((long long)S * H >= (1ll << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len * n_heads = %lld is too large", (long long)S * H);
  // byte offsets inside one staged 64-row tile must fit the 32-bit buffer offsets
  if ((long long)H * d >= (1ll << 23))
    return fail(ATTN_ERR_UNSUPPORTED, "n_heads * head_dim = %lld is too large", (long long)H * d);
  return ATTN_OK;
}

attn_status_t hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

// With stored tiles (a.scratch set): k_dq storing P and P*dP and emitting D,
// k_dkdv_p (dK, dV, and dS over P*dP), then k_dqs (dQ).  Without: k_dq
// accumulating dQ and emitting D, then k_dkdv recomputing the scores.  DK:
// D was computed beforehand (from the forward output); k_dq then stores
// dS/scale in place of P*dP, or accumulates dQ from dS alone.
template <int DP, bool DK>
static attn_status_t launch_dqkv(const BwdArgs& a, hipStream_t st, bool first) {
  // paired (plain causal): block p serves tile p and its mirror, so each grid halves
  auto blocks = [&](int ntiles) { return a.pair ? (ntiles + 1) / 2 : ntiles; };
  const int BRq = Pair<DP>::ROLE ? 64 : 128;
  const int nqt = blocks((a.S + BRq - 1) / BRq);
  attn_status_t rc = first ? profile_mark(st, true) : ATTN_OK;
  if (rc != ATTN_OK) return rc;
  if (a.scratch && DP > 128)
    hipLaunchKernelGGL((k_dqw<DP, DK>), dim3(nqt * a.H), dim3(256), 0, st, a);
  else if (a.scratch)
    hipLaunchKernelGGL((k_dq<DP, false, DK>), dim3(nqt * a.H), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_dq<DP, true, DK>), dim3(nqt * a.H), dim3(256), 0, st, a);
  rc = hip_check(hipGetLastError(), "launching k_dq");
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc != ATTN_OK) return rc;
  const int nkt = blocks((a.S + 63) / 64);
  if (a.scratch)
    hipLaunchKernelGGL((k_dkdv_p<DP, DK>), dim3(nkt * a.hsplit * a.KV), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_dkdv<DP>, dim3(nkt * a.KV), dim3(256), 0, st, a);
  rc = hip_check(hipGetLastError(), "launching the dK/dV kernel");
  if (rc == ATTN_OK && a.scratch && a.hsplit > 1)
    rc = launch_sumparts(a.part, a.hsplit - 1, a.S, a.KV * a.d, (long long)a.KVs * a.d, a.dK,
                         a.dV, st);
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc != ATTN_OK || !a.scratch) return rc;
  const int BRs = DP > 128 ? 64 : 128;
  hipLaunchKernelGGL(k_dqs<DP>, dim3(blocks((a.S + BRs - 1) / BRs) * a.H), dim3(256), 0, st, a);
  rc = hip_check(hipGetLastError(), "launching k_dqs");
  if (rc == ATTN_OK) rc = profile_mark(st);
  return rc;
}

template <bool DK>
static attn_status_t launch_bwd(const BwdArgs& a, int dp, hipStream_t st, bool first) {
  switch (dp) {
    case 32: return launch_dqkv<32, DK>(a, st, first);
    case 64: return launch_dqkv<64, DK>(a, st, first);
    case 96: return launch_dqkv<96, DK>(a, st, first);
    case 128: return launch_dqkv<128, DK>(a, st, first);
    case 192: return launch_dqkv<192, DK>(a, st, first);
    default: return launch_dqkv<256, DK>(a, st, first);
  }
}

// The library's own stream-ordered memory pool for the per-call workspaces.
// Freed workspace stays in the pool for later calls, up to ATTN_POOL_KEEP
// bytes (so a call of S=4096 with 32 heads, 2 GiB, maps nothing new after the
// first); the pool returns whatever it holds above that to the device at the
// caller's next synchronisation (its release threshold).  One pool per
// device, created on first use.
#define ATTN_POOL_KEEP (4ull << 30)
static std::mutex g_pool_mu;
static std::map<int, hipMemPool_t> g_pools;

attn_status_t device_pool(hipMemPool_t* out) {
  int dev = 0;
  attn_status_t rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != ATTN_OK) return rc;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  auto it = g_pools.find(dev);
  if (it != g_pools.end()) {
    *out = it->second;
    return ATTN_OK;
  }
  hipMemPoolProps props = {};
  props.allocType = hipMemAllocationTypePinned;
  props.location.type = hipMemLocationTypeDevice;
  props.location.id = dev;
  hipMemPool_t pool;
  rc = hip_check(hipMemPoolCreate(&pool, &props), "hipMemPoolCreate");
  if (rc != ATTN_OK) return rc;
  uint64_t keep = ATTN_POOL_KEEP;
  rc = hip_check(hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep),
                 "hipMemPoolSetAttribute");
  if (rc != ATTN_OK) return rc;
  g_pools[dev] = pool;
  *out = pool;
  return ATTN_OK;
}

// Bytes the P / P*dP scratch can need: at most qb + 1 key blocks per query
// block qb (the causal triangle; a document mask only shrinks it), two 4 KiB
// tiles per (block pair, head).
static long long scratch_bound(long long nblk, int H) {
  return nblk * (nblk + 1) / 2 * H * ATTN_TILE_FLOATS * (long long)sizeof(float);
}

// The most bytes of stored tiles one call may take (attn_set_scratch_limit).
static std::atomic<long long> g_scratch_limit{32ll << 30};

long long scratch_limit() { return g_scratch_limit.load(); }

extern "C" attn_status_t attn_set_scratch_limit(size_t bytes, size_t* previous) {
  g_err[0] = 0;
  const long long v = bytes > (size_t)LLONG_MAX ? LLONG_MAX : (long long)bytes;
  const long long old = g_scratch_limit.exchange(v);
  if (previous) *previous = (size_t)old;
  return ATTN_OK;
}

// How attn_bwd runs a problem.  The stored P / P*dP tiles are taken for
// `chunk` heads at a time: all heads when their causal bound fits the limit,
// else as many whole KV groups as fit, else the largest divisor of a group's
// size that fits (the chunks then run one after another, each adding its
// share into dK, dV); when not even one head's tiles fit, the key-major pass
// recomputes the scores instead (chunk = n_heads, nothing stored).  hsplit:
// how many workgroups share a key tile's heads in k_dkdv_p (the most any
// chunk takes).  Workspace layout: D [S, H], per-block seg min/max and slot
// offsets, the scratch of one chunk, then the partial dK, dV of the head
// splits after the first ([S, KV, d] slices).
struct Plan {
  bool stored = false;
  int chunk = 0;
  int hsplit = 1;
  size_t off_blk = 0, off_slot = 0, off_scr = 0, off_part = 0, bytes = 0;
};

// Heads per chunk when `fit` heads' tiles fit the limit (0: none).
static int chunk_heads(int H, int KV, long long fit) {
  const int g = H / KV;
  if (fit >= H) return H;
  if (fit >= g) return (int)(fit / g) * g;
  for (int c = (int)fit; c >= 1; --c)
    if (g % c == 0) return c;
  return 0;
}

// Unpaired calls (a seg given): paired tiles carry equal work; unpaired,
// under a document mask, the first key tile of a long document can hold more
// work than a CU's share of the whole pass, so k_dkdv_p splits each group's
// heads over workgroups until the launch has ~2048 of them (S=16384, 2 KV
// heads, documents: the longest workgroup came down from 1.3 to 1.12 times
// the mean load of a CU at ~1024; 4 splits instead of 2 then took k_dkdv_p
// from 4.44 to 4.18 ms, 8 splits 4.28 ms).  Hc heads over KVc KV heads in
// this launch.
static int head_splits(int S, int Hc, int KVc) {
  const long long blocks = ((long long)S + 63) / 64 * KVc;
  const int gc = Hc / KVc;
  int hs = 1;
  while (blocks * hs < 2048 && gc % (2 * hs) == 0) hs *= 2;
  return hs;
}

static Plan make_plan(int S, int H, int KV, int d, bool may_split, long long limit) {
  Plan p;
  const long long nblk = ((long long)S + 31) / 32;
  const long long per_head = scratch_bound(nblk, 1);
  // tile indices (slot * heads + head) stay below 2^31
  const long long budget = std::min(limit, 0x7fffffffll * ATTN_TILE_FLOATS * 4);
  p.chunk = per_head > 0 ? chunk_heads(H, KV, budget / per_head) : 0;
  p.stored = p.chunk > 0;
  if (!p.stored) p.chunk = H;
  const long long need = p.stored ? per_head * p.chunk : 0;
  const size_t nD = (size_t)S * H;
  p.off_blk = (nD * sizeof(float) + 255) & ~(size_t)255;
  p.off_slot = (p.off_blk + 2 * nblk * sizeof(uint32_t) + 255) & ~(size_t)255;
  p.off_scr = (p.off_slot + (nblk + 1) * sizeof(long long) + 255) & ~(size_t)255;
  p.off_part = (p.off_scr + (size_t)need + 255) & ~(size_t)255;
  if (p.stored && may_split) {
    const int g = H / KV;
    const int last = H % p.chunk ? H % p.chunk : p.chunk;  // a smaller last chunk
    p.hsplit = std::max(head_splits(S, p.chunk, std::max(1, p.chunk / g)),
                        head_splits(S, last, std::max(1, last / g)));
  }
  p.bytes = p.hsplit > 1 ? p.off_part + (size_t)2 * (p.hsplit - 1) * S * KV * d * sizeof(float)
                         : p.off_scr + (size_t)need;
  return p;
}

extern "C" attn_status_t attn_bwd_plan(int seq_len, int n_heads, int n_kv_heads, int head_dim,
                                       size_t* workspace_bytes, int* stored_heads) {
  g_err[0] = 0;
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, 1.f);
  if (rc != ATTN_OK) return rc;
  // the most a call of this size takes: an unpaired one, with head splits
  const Plan p = make_plan(seq_len, n_heads, n_kv_heads, head_dim, true, g_scratch_limit.load());
  if (workspace_bytes) *workspace_bytes = seq_len ? p.bytes : 0;
  if (stored_heads) *stored_heads = p.stored ? p.chunk : 0;
  return ATTN_OK;
}

template <int DP>
static attn_status_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.S + 127) / 128;
  if (a.O)
    hipLaunchKernelGGL((k_fwd<DP, true>), dim3(nqt * a.H), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_fwd<DP, false>), dim3(nqt * a.H), dim3(256), 0, st, a);
  return hip_check(hipGetLastError(), "launching k_fwd");
}

attn_status_t launch_prep(const uint32_t* seg, int S, uint32_t* blk_min, uint32_t* blk_max,
                          long long* slot_off, hipStream_t st) {
  hipLaunchKernelGGL(k_prep, dim3(1), dim3(1024), 0, st, seg, S, blk_min, blk_max, slot_off);
  return hip_check(hipGetLastError(), "launching k_prep");
}

attn_status_t launch_sumparts(const float* part, int splits, long long rows, int width,
                              long long stride, float* dK, float* dV, hipStream_t st, int rope,
                              int d, int rope_pos, double rope_base) {
  int tpr = 1;
  while (tpr < width / 4 && tpr < 256) tpr <<= 1;
  const int blocks = (int)std::min<long long>((rows + 256 / tpr - 1) / (256 / tpr), 8192);
  hipLaunchKernelGGL(k_sumparts, dim3(blocks), dim3(256), 0, st, part, splits, rows, width, stride,
                     dK, dV, rope, d, rope_pos, rope_base);
  return hip_check(hipGetLastError(), "launching k_sumparts");
}

attn_status_t launch_rowdot(const float* O, const float* dO, float* D, long long rows, int d,
                            hipStream_t st) {
  int tpr = 1;
  while (tpr < d / 4) tpr <<= 1;
  const long long waves = (rows * tpr + 63) / 64;
  const int blocks = (int)std::min<long long>((waves + 3) / 4, 4096);
  hipLaunchKernelGGL(k_rowdot, dim3(blocks), dim3(256), 0, st, O, dO, D, rows, d);
  return hip_check(hipGetLastError(), "launching k_rowdot");
}

// The backward on a planned workspace `wsb` (pl.bytes): the block metadata,
// D from the forward output when O is given, then the passes, in head chunks
// when the plan stores tiles for fewer than all heads.  rope: dQ and dK are
// rotated back in the write-back (rope_bwd).
static attn_status_t run_planned(const float* Q, const float* K, const float* V, const float* O,
                                 const float* dO, const float* LSE, const uint32_t* seg,
                                 float* dQ, float* dK, float* dV, int S, int H, int KV, int d,
                                 float scale, const Plan& pl, char* wsb, hipStream_t st, int rope,
                                 float rope_base, int pos_offset) {
  const long long nblk = ((long long)S + 31) / 32;
  BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.LSE = LSE; a.seg = seg;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Dws = reinterpret_cast<float*>(wsb);
  a.blk_min = reinterpret_cast<uint32_t*>(wsb + pl.off_blk);
  a.blk_max = a.blk_min + nblk;
  a.slot_off = reinterpret_cast<long long*>(wsb + pl.off_slot);
  a.scratch = pl.stored ? reinterpret_cast<float*>(wsb + pl.off_scr) : nullptr;
  a.S = S; a.H = H; a.KV = KV; a.d = d; a.scale = scale;
  a.Hs = H; a.KVs = KV;
  // plain causal: every tile's work falls linearly with its index, so a tile
  // and its mirror sum to the same work
  a.pair = seg == nullptr;
  a.hsplit = 1;
  a.part = pl.hsplit > 1 ? reinterpret_cast<float*>(wsb + pl.off_part) : nullptr;
  a.rope = rope;
  a.rope_old = 1;
  a.rope_pos = pos_offset;
  a.rope_base = (double)rope_base;

  const int dp = padded_dim(d);
  attn_status_t rc = launch_prep(seg, S, a.blk_min, a.blk_max, a.slot_off, st);
  if (rc == ATTN_OK && O) rc = launch_rowdot(O, dO, a.Dws, (long long)S * H, d, st);
  const int g = H / KV;
  for (int h0 = 0; h0 < H && rc == ATTN_OK; h0 += pl.chunk) {
    // heads [h0, h0 + hn) over KV heads [kv0, kv0 + c.KV): whole groups, or
    // a share of one group's heads (the chunk then divides the group)
    const int hn = std::min(pl.chunk, H - h0), kv0 = h0 / g;
    BwdArgs c = a;
    c.H = hn;
    c.KV = std::max(1, hn / g);
    c.Q = Q + (size_t)h0 * d; c.dO = dO + (size_t)h0 * d; c.dQ = dQ + (size_t)h0 * d;
    c.LSE = LSE + h0; c.Dws = a.Dws + h0;
    c.K = K + (size_t)kv0 * d; c.V = V + (size_t)kv0 * d;
    c.dK = dK + (size_t)kv0 * d; c.dV = dV + (size_t)kv0 * d;
    c.rope_old = h0 % g == 0;  // later shares of a group add to rotated dK rows
    if (pl.hsplit > 1) {
      c.hsplit = std::min(pl.hsplit, head_splits(S, c.H, c.KV));
      c.part = a.part + (size_t)kv0 * d;
    }
    rc = O ? launch_bwd<true>(c, dp, st, h0 == 0) : launch_bwd<false>(c, dp, st, h0 == 0);
  }
  return rc;
}

// The backward, with D computed by the kernels (O == NULL) or read off the
// forward output O, on a workspace from the library's pool.  If the pool
// cannot supply the stored-tile workspace (the device is out of memory), the
// call runs the recompute path, which needs only D and the block metadata.
static attn_status_t run_bwd(const float* Q, const float* K, const float* V, const float* O,
                             const float* dO, const float* LSE, const uint32_t* seg, float* dQ,
                             float* dK, float* dV, int seq_len, int n_heads, int n_kv_heads,
                             int head_dim, float scale, void* stream, int rope = 0,
                             float rope_base = 0.f, int pos_offset = 0) {
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, O, dO, LSE, seg, dQ, dK, dV};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len == 0) return ATTN_OK;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Plan pl = make_plan(seq_len, n_heads, n_kv_heads, head_dim, seg != nullptr,
                      g_scratch_limit.load());
  hipMemPool_t pool;
  rc = device_pool(&pool);
  if (rc != ATTN_OK) return rc;
  void* ws = nullptr;
  hipError_t e = hipMallocFromPoolAsync(&ws, pl.bytes, pool, st);
  if (e == hipErrorOutOfMemory && pl.stored) {
    (void)hipGetLastError();  // the failed allocation is not a launch error
    pl = make_plan(seq_len, n_heads, n_kv_heads, head_dim, seg != nullptr, 0);
    e = hipMallocFromPoolAsync(&ws, pl.bytes, pool, st);
  }
  rc = hip_check(e, "hipMallocFromPoolAsync(workspace)");
  if (rc != ATTN_OK) return rc;
  rc = run_planned(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                   scale, pl, static_cast<char*>(ws), st, rope, rope_base, pos_offset);
  attn_status_t rc2 = hip_check(hipFreeAsync(ws, st), "hipFreeAsync(workspace)");
  return rc != ATTN_OK ? rc : rc2;
}

// ---------------------------------------------------------------------------
// The entry that allocates nothing (attn_bwd_noalloc): its workspace is this
// file-scope device array, one per device, held from the library's load on
// that device until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): it looks up the array's device address once per device and passes
// that.
// ---------------------------------------------------------------------------
#define ATTN_NOALLOC_BYTES (32u << 20)
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_BYTES];
static std::mutex g_scratch_mu;
static std::map<int, char*> g_scratch_ptr;

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current).
static attn_status_t noalloc_scratch(char** out) {
  int dev = 0;
  attn_status_t rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != ATTN_OK) return rc;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return ATTN_OK;
  }
  void* ptr = nullptr;
  rc = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
  if (rc != ATTN_OK) return rc;
  g_scratch_ptr[dev] = static_cast<char*>(ptr);
  *out = static_cast<char*>(ptr);
  return ATTN_OK;
}

// A plan whose workspace fits `avail` bytes: the stored tiles of as many heads
// as fit beside D and the metadata (head splits first allowed, then not),
// else the recompute path; false when not even D and the metadata fit.
static bool plan_within(int S, int H, int KV, int d, bool may_split, size_t avail, Plan* out) {
  for (int split = may_split ? 1 : 0; split >= 0; --split) {
    long long limit = (long long)avail;
    for (int it = 0; it < 64; ++it) {
      const Plan p = make_plan(S, H, KV, d, split != 0, limit);
      if (p.bytes <= avail) {
        *out = p;
        return true;
      }
      if (!p.stored) break;
      limit = std::max(0ll, limit - (long long)(p.bytes - avail));  // shrink by the excess
    }
  }
  return false;
}

extern "C" attn_status_t attn_bwd_noalloc(const float* Q, const float* K, const float* V,
                                          const float* dO, const float* LSE, const uint32_t* seg,
                                          float* dQ, float* dK, float* dV, int seq_len,
                                          int n_heads, int n_kv_heads, int head_dim, float scale,
                                          void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, dO, LSE, seg, dQ, dK, dV};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len == 0) return ATTN_OK;
  Plan pl;
  if (!plan_within(seq_len, n_heads, n_kv_heads, head_dim, seg != nullptr, ATTN_NOALLOC_BYTES, &pl))
    return fail(ATTN_ERR_UNSUPPORTED,
                "attn_bwd_noalloc: seq_len %d with %d heads needs more than its %u-byte scratch "
                "(the row term alone is seq_len * n_heads * 4 bytes)",
                seq_len, n_heads, ATTN_NOALLOC_BYTES);
  char* ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc != ATTN_OK) return rc;
  return run_planned(Q, K, V, nullptr, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads,
                     head_dim, scale, pl, ws, reinterpret_cast<hipStream_t>(stream), 0, 0.f, 0);
}

extern "C" attn_status_t attn_bwd(const float* Q, const float* K, const float* V, const float* dO,
                                  const float* LSE, const uint32_t* seg, float* dQ, float* dK,
                                  float* dV, int seq_len, int n_heads, int n_kv_heads,
                                  int head_dim, float scale, void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  return run_bwd(Q, K, V, nullptr, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads,
                 head_dim, scale, stream);
}

extern "C" attn_status_t attn_bwd_o(const float* Q, const float* K, const float* V,
                                    const float* O, const float* dO, const float* LSE,
                                    const uint32_t* seg, float* dQ, float* dK, float* dV,
                                    int seq_len, int n_heads, int n_kv_heads, int head_dim,
                                    float scale, void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  return run_bwd(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                 scale, stream);
}

extern "C" attn_status_t attn_bwd_rope(const float* Q, const float* K, const float* V,
                                       const float* O, const float* dO, const float* LSE,
                                       const uint32_t* seg, float* dQ, float* dK, float* dV,
                                       int seq_len, int n_heads, int n_kv_heads, int head_dim,
                                       float scale, float rope_base, int pos_offset,
                                       void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (!(rope_base > 0.f) || !isfinite(rope_base))
    return fail(ATTN_ERR_INVALID_ARG, "rope_base must be positive and finite (got %g)", (double)rope_base);
  if (pos_offset < 0) return fail(ATTN_ERR_INVALID_ARG, "pos_offset must be >= 0 (got %d)", pos_offset);
  if (seq_len > 0 && (long long)pos_offset + seq_len - 1 > 0x7fffffffll)
    return fail(ATTN_ERR_INVALID_ARG, "pos_offset + seq_len exceeds 2^31");
  return run_bwd(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                 scale, stream, 1, rope_base, pos_offset);
}

extern "C" attn_status_t attn_fwd_lse(const float* Q, const float* K, const float* V,
                                      const uint32_t* seg, float* O, float* LSE, int seq_len,
                                      int n_heads, int n_kv_heads, int head_dim, float scale,
                                      void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !LSE) return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, seg, O, LSE};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len == 0) return ATTN_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.seg = seg; a.O = O; a.LSE = LSE;
  a.S = seq_len; a.H = n_heads; a.KV = n_kv_heads; a.d = head_dim; a.scale = scale;
  switch (padded_dim(head_dim)) {
    case 32: return launch_fwd<32>(a, st);
    case 64: return launch_fwd<64>(a, st);
    case 96: return launch_fwd<96>(a, st);
    case 128: return launch_fwd<128>(a, st);
    case 192: return launch_fwd<192>(a, st);
    default: return launch_fwd<256>(a, st);
  }
}
