// attnbwd.hip -- causal grouped-query attention backward with a per-query
// document-start mask, for CDNA4 (gfx950 / MI355X), fp32 in and out, fp32
// matrix-core (MFMA) arithmetic.
//
// Operation: page "llm.istanbul -- 10_backward_attention.wgsl", header
// comment and kernel attention_backward (Pass A: P, dP, D and dV; Pass B: dS,
// dQ and dK; Final: owned += of dQ).  The page's design (one workgroup per
// (query, head), CAS-atomic dK/dV scatter) was made for WebGPU on Apple GPUs;
// here the same sums are re-tiled for 64-wide wavefronts and MFMA:
//
//   k_dq   query-block-major.  One workgroup per (query tile, head).  Sweeps
//          the visible key tiles once and accumulates, per query row,
//             A = sum_j P*dP*k_j     B = sum_j P*k_j     D = sum_j P*dP
//          so dQ = scale*(A - D*B) (= sum_j dS*k_j), and D is emitted for k_dkdv.
//          4 MFMA contractions per visible pair: K.Q^T, V.dO^T, (P.dP).K, P.K.
//   k_dkdv key-block-major.  One workgroup per (key tile, KV head).  Owns its
//          dK/dV rows, sums the GQA group inside the workgroup (the key-major,
//          atomic-free idea of the page's attention_backward_short_dKdV
//          kernel), sweeps the query tiles that can see its keys.
//          4 MFMA contractions per visible pair: Q.K^T, dO.V^T, P^T.dO, dS^T.Q.
//   k_fwd  forward producing LSE (and optionally O) for the backward's input
//          (page "tang 0.2.0 -- src/gpu/llm.rs", causal_attention_fused: row
//          max, exp-sum, weighted V; plus the document mask and the LSE output).
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

#include <vector>

#include "attnbwd.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));

#define ATTN_LOG2E 1.4426950408889634f
#define ATTN_LN2 0.6931471805599453f

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// row of a 32x32 accumulator tile held in register r by half-wave hf
__device__ __forceinline__ int crow(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Geometry shared by the kernels for a padded head dimension DP (a multiple of
// 32; head_dim is zero-padded up to it).  Above 128 columns the contraction
// over d is split between a pair of waves (DSPL = 2) that exchange partial
// score tiles through LDS, so that each wave keeps DP/2 columns in registers.
template <int DP>
struct Geo {
  static constexpr int DSPL = DP > 128 ? 2 : 1;
  static constexpr int DW = DP / DSPL;  // columns owned by one wave
  static constexpr int TH = DW / 2;     // contraction steps per half-wave
  static constexpr int NB = DW / 32;    // 32-column output blocks per wave
  static constexpr int LDR = DP + 4;    // LDS row stride in floats (b128 reads conflict-free)
  static_assert(DW % 32 == 0, "a wave owns whole 32-column blocks");
};

struct BwdArgs {
  const float *Q, *K, *V, *dO, *LSE;
  const uint32_t* seg;  // NULL = all zeros
  float *dQ, *dK, *dV;
  float* Dws;            // [S, H] row term, written by k_dq, read by k_dkdv
  uint32_t* blk_min;     // [ceil(S/32)] min seg per 32-row query block
  int S, H, KV, d;
  float scale;
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

// Cooperative load of ROWS x DP floats of two row-major matrices that share
// addressing (K and V, or Q and dO) into registers, one float4 per step.
template <int ROWS, int DP>
struct TilePair {
  static constexpr int F4 = ROWS * DP / 4 / 256;
  static_assert(F4 * 256 * 4 == ROWS * DP, "tile must split evenly over 256 threads");
  float4 a[F4], b[F4];

  __device__ __forceinline__ void fetch(const float* A, const float* B, int r0, int S,
                                        size_t row_stride, size_t col0, int d, int tid) {
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int f = tid + 256 * i;
      const int row = f / (DP / 4), col = (f % (DP / 4)) * 4;
      a[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      b[i] = a[i];
      if (r0 + row < S && col < d) {
        const size_t off = (size_t)(r0 + row) * row_stride + col0 + col;
        a[i] = *reinterpret_cast<const float4*>(A + off);
        b[i] = *reinterpret_cast<const float4*>(B + off);
      }
    }
  }
  __device__ __forceinline__ void stash(float* sA, float* sB, int tid) const {
    constexpr int LDR = DP + 4;
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int f = tid + 256 * i;
      const int row = f / (DP / 4), col = (f % (DP / 4)) * 4;
      *reinterpret_cast<float4*>(sA + row * LDR + col) = a[i];
      *reinterpret_cast<float4*>(sB + row * LDR + col) = b[i];
    }
  }
};

// Exchange of partial score tiles between the two waves of a d-split pair:
// each adds its partner's partial sums (a + b in one wave, b + a in the other,
// so both hold bitwise identical tiles).
__device__ __forceinline__ void pair_exchange(float* sX, int wave, int lane, f32x16& x, f32x16& y) {
  float* mine = sX + (wave * 32) * 64 + lane;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mine[r * 64] = x[r];
    mine[(16 + r) * 64] = y[r];
  }
  __syncthreads();
  const float* other = sX + ((wave ^ 1) * 32) * 64 + lane;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] += other[r * 64];
    y[r] += other[(16 + r) * 64];
  }
}

// ---------------------------------------------------------------------------
// k_dq: D and dQ, one workgroup per (query tile of BR rows, head).
// Wave w owns query block qb = w / DSPL (32 queries) and contraction half
// ds = w % DSPL.  Key tiles of 32 rows of K and V are staged in LDS,
// double-buffered through registers.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void k_dq(BwdArgs a) {
  using G = Geo<DP>;
  constexpr int QB = 4 / G::DSPL, BR = 32 * QB, BC = 32;
  __shared__ __attribute__((aligned(16))) float sK[BC * G::LDR];
  __shared__ __attribute__((aligned(16))) float sV[BC * G::LDR];
  __shared__ __attribute__((aligned(16))) float sX[G::DSPL > 1 ? 4 * 32 * 64 : 4];
  __shared__ float sD[4 * 32];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int ds = wave % G::DSPL, qb = wave / G::DSPL;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int nqt = (S + BR - 1) / BR;
  const int qt = nqt - 1 - (int)(blockIdx.x / H);  // longest rows first
  const int h = blockIdx.x % H, kvh = h / g;
  const int i0 = qt * BR;
  const int q = i0 + qb * 32 + l32;
  const bool q_ok = q < S;
  const int cb = ds * G::DW + hf * G::TH;
  const size_t qstride = (size_t)H * d, kstride = (size_t)a.KV * d;
  const float sc2 = a.scale * ATTN_LOG2E;

  float qr[G::TH], gr[G::TH];
  load_row<G::TH>(a.Q + (size_t)q * qstride + (size_t)h * d, cb, d, q_ok, qr);
  load_row<G::TH>(a.dO + (size_t)q * qstride + (size_t)h * d, cb, d, q_ok, gr);
  const float lse2 = q_ok ? a.LSE[(size_t)q * H + h] * ATTN_LOG2E : 0.f;
  const uint32_t sq = (q_ok && a.seg) ? a.seg[q] : 0u;

  // smallest document start of the tile bounds the key sweep
  uint32_t mn = q_ok ? sq : 0xffffffffu;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
  if (lane == 0) sMin[wave] = mn;
  __syncthreads();
  uint32_t tmin = sMin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tmin = min(tmin, sMin[w]);
  if (h == 0 && ds == 0 && lane == 0 && i0 + qb * 32 < S) a.blk_min[(i0 >> 5) + qb] = mn;

  const int last_q = min(i0 + BR, S) - 1;
  const int kt_lo = (int)(min(tmin, (uint32_t)last_q) / BC), kt_hi = last_q / BC;

  f32x16 accA[G::NB], accB[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) { accA[nb] = zero16(); accB[nb] = zero16(); }
  float Dp = 0.f;

  TilePair<BC, DP> pf;
  pf.fetch(a.K, a.V, kt_lo * BC, S, kstride, (size_t)kvh * d, d, tid);
  pf.stash(sK, sV, tid);
  __syncthreads();

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const bool more = kt < kt_hi;
    if (more) pf.fetch(a.K, a.V, (kt + 1) * BC, S, kstride, (size_t)kvh * d, d, tid);
    const int j0 = kt * BC;

    // S^T = K Q^T and dP^T = V dO^T for 32 keys x this wave's 32 queries
    f32x16 st = zero16(), dpt = zero16();
    const float* kp = sK + l32 * G::LDR + cb;
    const float* vp = sV + l32 * G::LDR + cb;
#pragma unroll
    for (int t = 0; t < G::TH; t += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(kp + t);
      const float4 v4 = *reinterpret_cast<const float4*>(vp + t);
      st = mfma32(k4.x, qr[t], st);
      dpt = mfma32(v4.x, gr[t], dpt);
      st = mfma32(k4.y, qr[t + 1], st);
      dpt = mfma32(v4.y, gr[t + 1], dpt);
      st = mfma32(k4.z, qr[t + 2], st);
      dpt = mfma32(v4.z, gr[t + 2], dpt);
      st = mfma32(k4.w, qr[t + 3], st);
      dpt = mfma32(v4.w, gr[t + 3], dpt);
    }
    if constexpr (G::DSPL > 1) pair_exchange(sX, wave, lane, st, dpt);

    // P and P*dP in place; this lane's query, key = crow(r, hf)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + crow(r, hf);
      const bool vis = q_ok && key <= q && (uint32_t)key >= sq;
      const float e = exp2f(fmaf(st[r], sc2, -lse2));
      const float p = vis ? e : 0.f;
      const float pdp = vis ? p * dpt[r] : 0.f;
      Dp += pdp;
      st[r] = p;
      dpt[r] = pdp;
    }
    // A += (P.dP) K,  B += P K over the 32 keys (register r = key crow(r, hf))
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* krow = sK + crow(r, hf) * G::LDR + ds * G::DW + l32;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const float kb = krow[nb * 32];
        accB[nb] = mfma32(st[r], kb, accB[nb]);
        accA[nb] = mfma32(dpt[r], kb, accA[nb]);
      }
    }
    __syncthreads();
    if (more) {
      pf.stash(sK, sV, tid);
      __syncthreads();
    }
  }

  // D of this lane's query: the two half-waves saw disjoint keys
  const float Dq = Dp + __shfl_xor(Dp, 32);
  if (hf == 0) sD[wave * 32 + l32] = Dq;
  if (q_ok && hf == 0 && ds == 0) a.Dws[(size_t)q * H + h] = Dq;
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int col = ds * G::DW + nb * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = crow(r, hf);
      const int row = i0 + qb * 32 + m;
      if (row < S && col < d) {
        float* o = a.dQ + (size_t)row * qstride + (size_t)h * d + col;
        *o += a.scale * (accA[nb][r] - sD[wave * 32 + m] * accB[nb][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_dkdv: dK and dV, one workgroup per (key tile of BC = 64 rows, KV head).
// Wave w: key block kb (32 keys), query split qs, contraction half ds.  K and
// V of the wave's keys live in registers; Q/dO tiles of BR rows of each head
// of the group are staged in LDS.  Partial dK/dV of the QS query splits are
// summed through LDS at the end; each (key, KV head) row has one writer.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void k_dkdv(BwdArgs a) {
  using G = Geo<DP>;
  constexpr int KB = 2, QS = 2 / G::DSPL, BC = 32 * KB, BR = 32 * QS;
  constexpr int TILE = BR * G::LDR;
  static_assert(QS == 1 || 2 * TILE >= KB * 2 * G::NB * 16 * 64, "reduction buffer fits");
  __shared__ __attribute__((aligned(16))) float sQG[2 * TILE];
  __shared__ float sL[BR], sDD[BR];
  __shared__ uint32_t sS[BR];
  __shared__ __attribute__((aligned(16))) float sX[G::DSPL > 1 ? 4 * 32 * 64 : 4];
  float* sQ = sQG;
  float* sG = sQG + TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int ds = wave % G::DSPL, rest = wave / G::DSPL;
  const int qs = rest % QS, kb = rest / QS;
  const int S = a.S, H = a.H, KV = a.KV, d = a.d;
  const int g = H / KV;
  const int kt = blockIdx.x / KV, kvh = blockIdx.x % KV;  // low key tiles (most queries) first
  const int j0 = kt * BC;
  const int key = j0 + kb * 32 + l32;
  const bool key_ok = key < S;
  const int cb = ds * G::DW + hf * G::TH;
  const size_t qstride = (size_t)H * d, kstride = (size_t)KV * d;
  const float sc2 = a.scale * ATTN_LOG2E;

  float kr[G::TH], vr[G::TH];
  load_row<G::TH>(a.K + (size_t)key * kstride + (size_t)kvh * d, cb, d, key_ok, kr);
  load_row<G::TH>(a.V + (size_t)key * kstride + (size_t)kvh * d, cb, d, key_ok, vr);

  f32x16 accK[G::NB], accV[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) { accK[nb] = zero16(); accV[nb] = zero16(); }

  const int jlast = min(j0 + BC, S) - 1;
  const int nqt = (S + BR - 1) / BR, qt0 = j0 / BR;
  const int nblk = (S + 31) / 32;

  for (int hh = 0; hh < g; ++hh) {
    const int h = kvh * g + hh;
    for (int qt = qt0; qt < nqt; ++qt) {
      const int i0 = qt * BR;
      uint32_t mn = 0xffffffffu;
#pragma unroll
      for (int b = 0; b < QS; ++b) {
        const int bi = (i0 >> 5) + b;
        if (bi < nblk) mn = min(mn, a.blk_min[bi]);
      }
      if (mn > (uint32_t)jlast) continue;  // no query of the tile sees these keys

      TilePair<BR, DP> t;
      t.fetch(a.Q, a.dO, i0, S, qstride, (size_t)h * d, d, tid);
      t.stash(sQ, sG, tid);
      if (tid < BR) {
        const int s = i0 + tid;
        const bool ok = s < S;
        sL[tid] = ok ? a.LSE[(size_t)s * H + h] * ATTN_LOG2E : 0.f;
        sDD[tid] = ok ? a.Dws[(size_t)s * H + h] : 0.f;
        sS[tid] = ok ? (a.seg ? a.seg[s] : 0u) : 0xffffffffu;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys
      f32x16 s = zero16(), dp = zero16();
      const float* qp = sQ + (qs * 32 + l32) * G::LDR + cb;
      const float* gp = sG + (qs * 32 + l32) * G::LDR + cb;
#pragma unroll
      for (int t4 = 0; t4 < G::TH; t4 += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(qp + t4);
        const float4 g4 = *reinterpret_cast<const float4*>(gp + t4);
        s = mfma32(q4.x, kr[t4], s);
        dp = mfma32(g4.x, vr[t4], dp);
        s = mfma32(q4.y, kr[t4 + 1], s);
        dp = mfma32(g4.y, vr[t4 + 1], dp);
        s = mfma32(q4.z, kr[t4 + 2], s);
        dp = mfma32(g4.z, vr[t4 + 2], dp);
        s = mfma32(q4.w, kr[t4 + 3], s);
        dp = mfma32(g4.w, vr[t4 + 3], dp);
      }
      if constexpr (G::DSPL > 1) pair_exchange(sX, wave, lane, s, dp);

      // P and dS in place; register r = query qs*32 + crow(r, hf), lane = key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qs * 32 + crow(r, hf);
        const int qi = i0 + row;
        const bool vis = key <= qi && sS[row] <= (uint32_t)key && qi < S;
        const float e = exp2f(fmaf(s[r], sc2, -sL[row]));
        const float p = vis ? e : 0.f;
        const float dsv = vis ? a.scale * p * (dp[r] - sDD[row]) : 0.f;
        s[r] = p;
        dp[r] = dsv;
      }
      // dV += P^T dO,  dK += dS^T Q over the 32 queries
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qs * 32 + crow(r, hf);
        const float* grow = sG + row * G::LDR + ds * G::DW + l32;
        const float* qrow = sQ + row * G::LDR + ds * G::DW + l32;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
          accV[nb] = mfma32(s[r], grow[nb * 32], accV[nb]);
          accK[nb] = mfma32(dp[r], qrow[nb * 32], accK[nb]);
        }
      }
      __syncthreads();
    }
  }

  if constexpr (QS > 1) {
    float* red = sQG + kb * (2 * G::NB * 16 * 64) + lane;
    if (qs == 1) {
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[((0 * G::NB + nb) * 16 + r) * 64] = accK[nb][r];
          red[((1 * G::NB + nb) * 16 + r) * 64] = accV[nb][r];
        }
    }
    __syncthreads();
    if (qs == 1) return;
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accK[nb][r] += red[((0 * G::NB + nb) * 16 + r) * 64];
        accV[nb][r] += red[((1 * G::NB + nb) * 16 + r) * 64];
      }
  }
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int col = ds * G::DW + nb * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = j0 + kb * 32 + crow(r, hf);
      if (row < S && col < d) {
        const size_t off = (size_t)row * kstride + (size_t)kvh * d + col;
        a.dK[off] += accK[nb][r];
        a.dV[off] += accV[nb][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_fwd: LSE (pass 1, running max and sum per query) and O (pass 2, with the
// final LSE, no rescaling).  Same tiling as k_dq.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void k_fwd(FwdArgs a) {
  using G = Geo<DP>;
  constexpr int QB = 4 / G::DSPL, BR = 32 * QB, BC = 32;
  __shared__ __attribute__((aligned(16))) float sK[BC * G::LDR];
  __shared__ __attribute__((aligned(16))) float sV[BC * G::LDR];
  __shared__ __attribute__((aligned(16))) float sX[G::DSPL > 1 ? 4 * 32 * 64 : 4];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int ds = wave % G::DSPL, qb = wave / G::DSPL;
  const int S = a.S, H = a.H, d = a.d;
  const int g = H / a.KV;
  const int nqt = (S + BR - 1) / BR;
  const int qt = nqt - 1 - (int)(blockIdx.x / H);
  const int h = blockIdx.x % H, kvh = h / g;
  const int i0 = qt * BR;
  const int q = i0 + qb * 32 + l32;
  const bool q_ok = q < S;
  const int cb = ds * G::DW + hf * G::TH;
  const size_t qstride = (size_t)H * d, kstride = (size_t)a.KV * d;
  const float sc2 = a.scale * ATTN_LOG2E;

  float qr[G::TH];
  load_row<G::TH>(a.Q + (size_t)q * qstride + (size_t)h * d, cb, d, q_ok, qr);
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

  float m = -INFINITY, l = 0.f;  // running max / sum (log2 domain) over this half's keys
  float lse2 = -INFINITY;
  f32x16 accO[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) accO[nb] = zero16();

  for (int pass = 0; pass < (a.O ? 2 : 1); ++pass) {
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      const int j0 = kt * BC;
      TilePair<BC, DP> t;
      t.fetch(a.K, a.V, j0, S, kstride, (size_t)kvh * d, d, tid);
      t.stash(sK, sV, tid);
      __syncthreads();
      f32x16 st = zero16(), unused = zero16();
      const float* kp = sK + l32 * G::LDR + cb;
#pragma unroll
      for (int t4 = 0; t4 < G::TH; t4 += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(kp + t4);
        st = mfma32(k4.x, qr[t4], st);
        st = mfma32(k4.y, qr[t4 + 1], st);
        st = mfma32(k4.z, qr[t4 + 2], st);
        st = mfma32(k4.w, qr[t4 + 3], st);
      }
      if constexpr (G::DSPL > 1) pair_exchange(sX, wave, lane, st, unused);
      if (pass == 0) {
        float x[16], mloc = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + crow(r, hf);
          const bool vis = q_ok && key <= q && (uint32_t)key >= sq;
          x[r] = vis ? st[r] * sc2 : -INFINITY;
          mloc = fmaxf(mloc, x[r]);
        }
        const float mnew = fmaxf(m, mloc);
        if (mnew != -INFINITY) {
          float acc = (m == -INFINITY) ? 0.f : l * exp2f(m - mnew);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += (x[r] == -INFINITY) ? 0.f : exp2f(x[r] - mnew);
          l = acc;
          m = mnew;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + crow(r, hf);
          const bool vis = q_ok && key <= q && (uint32_t)key >= sq;
          const float e = exp2f(fmaf(st[r], sc2, -lse2));
          st[r] = vis ? e : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* vrow = sV + crow(r, hf) * G::LDR + ds * G::DW + l32;
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) accO[nb] = mfma32(st[r], vrow[nb * 32], accO[nb]);
        }
      }
      __syncthreads();
    }
    if (pass == 0) {
      const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
      const float M = fmaxf(m, m2);
      if (M != -INFINITY) {
        const float L = ((m == -INFINITY) ? 0.f : l * exp2f(m - M)) +
                        ((m2 == -INFINITY) ? 0.f : l2 * exp2f(m2 - M));
        lse2 = M + log2f(L);
      }
      if (q_ok && hf == 0 && ds == 0) a.LSE[(size_t)q * H + h] = lse2 * ATTN_LN2;
    }
  }
  if (!a.O) return;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int col = ds * G::DW + nb * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i0 + qb * 32 + crow(r, hf);
      if (row < S && col < d) a.O[(size_t)row * qstride + (size_t)h * d + col] = accO[nb][r];
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static thread_local char g_err[512];

static attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

extern "C" const char* attn_last_error(void) { return g_err; }

// Per-thread event log of the measurement hooks (see attn_profile_begin).
struct ProfileLog {
  bool on = false;
  std::vector<hipEvent_t> ev;  // 3 per recorded attn_bwd call
};
static thread_local ProfileLog g_prof;

static void profile_release() {
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
}

extern "C" attn_status_t attn_profile_begin(void) {
  g_err[0] = 0;
  profile_release();
  g_prof.on = true;
  return ATTN_OK;
}

extern "C" attn_status_t attn_profile_end(double* ms, int* n_calls) {
  g_err[0] = 0;
  double sum[2] = {0.0, 0.0};
  attn_status_t rc = ATTN_OK;
  const size_t n = g_prof.ev.size() / 3;
  for (size_t i = 0; i < n && rc == ATTN_OK; ++i) {
    for (int k = 0; k < 2 && rc == ATTN_OK; ++k) {
      float t = 0.f;
      hipError_t e = hipEventSynchronize(g_prof.ev[3 * i + k + 1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof.ev[3 * i + k], g_prof.ev[3 * i + k + 1]);
      if (e != hipSuccess) rc = fail(ATTN_ERR_HIP, "reading profile events: %s", hipGetErrorString(e));
      sum[k] += t;
    }
  }
  if (ms) { ms[0] = sum[0]; ms[1] = sum[1]; }
  if (n_calls) *n_calls = (int)n;
  profile_release();
  g_prof.on = false;
  return rc;
}

// Record one profile event on `st` if the measurement hooks are on.
static attn_status_t profile_mark(hipStream_t st) {
  if (!g_prof.on) return ATTN_OK;
  hipEvent_t e;
  hipError_t err = hipEventCreate(&e);
  if (err == hipSuccess) err = hipEventRecord(e, st);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "profile event: %s", hipGetErrorString(err));
  g_prof.ev.push_back(e);
  return ATTN_OK;
}

static int padded_dim(int d) {
  if (d <= 32) return 32;
  if (d <= 64) return 64;
  if (d <= 96) return 96;
  if (d <= 128) return 128;
  if (d <= 192) return 192;
  return 256;
}

static bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

static attn_status_t check_common(int S, int H, int KV, int d, float scale) {
  if (S < 0) return fail(ATTN_ERR_INVALID_ARG, "seq_len = %d is negative", S);
  if (H < 1 || KV < 1) return fail(ATTN_ERR_INVALID_ARG, "n_heads = %d, n_kv_heads = %d", H, KV);
  if (H % KV != 0)
    return fail(ATTN_ERR_INVALID_ARG, "n_heads = %d is not a multiple of n_kv_heads = %d", H, KV);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
  if (d < 16 || d > 256 || d % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim = %d (supported: multiples of 16 in [16, 256])", d);
  if ((long long)S * H >= (1ll << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len * n_heads = %lld is too large", (long long)S * H);
  return ATTN_OK;
}

static attn_status_t hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

template <int DP>
static attn_status_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  constexpr int DSPL = Geo<DP>::DSPL;
  const int BRq = 32 * (4 / DSPL);
  const int nqt = (a.S + BRq - 1) / BRq;
  attn_status_t rc = profile_mark(st);
  if (rc != ATTN_OK) return rc;
  hipLaunchKernelGGL(k_dq<DP>, dim3(nqt * a.H), dim3(256), 0, st, a);
  rc = hip_check(hipGetLastError(), "launching k_dq");
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc != ATTN_OK) return rc;
  const int nkt = (a.S + 63) / 64;
  hipLaunchKernelGGL(k_dkdv<DP>, dim3(nkt * a.KV), dim3(256), 0, st, a);
  rc = hip_check(hipGetLastError(), "launching k_dkdv");
  if (rc == ATTN_OK) rc = profile_mark(st);
  return rc;
}

template <int DP>
static attn_status_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  const int BRq = 32 * (4 / Geo<DP>::DSPL);
  const int nqt = (a.S + BRq - 1) / BRq;
  hipLaunchKernelGGL(k_fwd<DP>, dim3(nqt * a.H), dim3(256), 0, st, a);
  return hip_check(hipGetLastError(), "launching k_fwd");
}

extern "C" attn_status_t attn_bwd(const float* Q, const float* K, const float* V, const float* dO,
                                  const float* LSE, const uint32_t* seg, float* dQ, float* dK,
                                  float* dV, int seq_len, int n_heads, int n_kv_heads,
                                  int head_dim, float scale, void* stream) {
  g_err[0] = 0;
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, dO, LSE, seg, dQ, dK, dV};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len == 0) return ATTN_OK;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t nD = (size_t)seq_len * n_heads;
  const size_t nblk = ((size_t)seq_len + 31) / 32;
  void* ws = nullptr;
  rc = hip_check(hipMallocAsync(&ws, nD * sizeof(float) + nblk * sizeof(uint32_t), st),
                 "hipMallocAsync(workspace)");
  if (rc != ATTN_OK) return rc;

  BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.LSE = LSE; a.seg = seg;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Dws = static_cast<float*>(ws);
  a.blk_min = reinterpret_cast<uint32_t*>(static_cast<float*>(ws) + nD);
  a.S = seq_len; a.H = n_heads; a.KV = n_kv_heads; a.d = head_dim; a.scale = scale;

  switch (padded_dim(head_dim)) {
    case 32: rc = launch_bwd<32>(a, st); break;
    case 64: rc = launch_bwd<64>(a, st); break;
    case 96: rc = launch_bwd<96>(a, st); break;
    case 128: rc = launch_bwd<128>(a, st); break;
    case 192: rc = launch_bwd<192>(a, st); break;
    default: rc = launch_bwd<256>(a, st); break;
  }
  attn_status_t rc2 = hip_check(hipFreeAsync(ws, st), "hipFreeAsync(workspace)");
  return rc != ATTN_OK ? rc : rc2;
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
