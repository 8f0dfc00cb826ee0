// attnbwd_decode.hip -- the single-query attention backward over a KV history
// (attn_bwd_decode): page "rullama 0.5.0 -- src/backend/dispatch/training.rs",
// attention_backward_dq_chained and attention_backward_dkv_chained (pass 1
// and pass 2 of 2).  One query per head (a decode step) attended to every
// key of a history of T positions, and the forward's probabilities P[h][j]
// are given, so nothing is recomputed:
//   dP[h][j] = dO_h . v_j,  D_h = sum_j P dP,  dS = P (dP - D)
//   dq_h += scale sum_j dS k_j;  dK_j += scale sum_{h in group} dS q_h;
//   dV_j += sum_{h in group} P dO_h.
// fp32 throughout.  Bound by HBM: every K, V, dK, dV element is read or
// written once or twice, against 2 multiply-adds per element per head.
//
// Passes (deterministic: every sum has one writer and a fixed order):
//   k_dec_dp  one workgroup per (128-key chunk, KV head), the KV heads of a
//             chunk adjacent in launch order (their rows of K, V, dK, dV are
//             one contiguous block): the group's dO rows in LDS, V rows
//             staged per wave 16 keys at a time, dP for (key, head) pairs one
//             lane each, stored; the chunk's partial row terms sum P dP.
//   k_dec_kv  same grid: D_h = the chunk partials summed in chunk order; dS in
//             LDS; dK and dV of the chunk's keys (coalesced over columns);
//             per-chunk partial dq sums.
//   k_dec_dq  dq += scale * the chunk partials summed in chunk order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

#define DEC_TB 128  // keys per chunk

// A 16-byte load that is marked nontemporal: the history's K, V, dK and dV
// rows are each read once per pass, so they are streamed past the caches
// (measured faster than plain loads for both passes; stores stay plain).
typedef float dec_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 stream_load(const float4* p) {
  const dec_f4 v = __builtin_nontemporal_load(reinterpret_cast<const dec_f4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

struct DecArgs {
  const float *q, *K, *V, *P, *dO;  // [H, d], [T, KV, d] x 2, [H, T], [H, d]
  float *dq, *dK, *dV;              // [H, d], [T, KV, d] x 2 (accumulated)
  float* dP;                        // [H, T] workspace
  float* partD;                     // [H, nch] workspace: sum_j P dP per chunk
  float* partQ;                     // [nch, H, d] workspace: sum_j dS k_j per chunk
  int T, H, KV, d, nch;
  float scale;
};

// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---------------------------------------------------------------------------
// k_dec_dp<NL>: per (chunk of 128 keys, KV head); the group's dO rows (16
// heads at a time) staged in LDS.  Wave w takes keys 32 w .. 32 w + 31 of the
// chunk in two steps of DEC_KW = 16: the step's V rows are loaded coalesced
// (NL = ceil(d / 16) 16-byte loads per lane) into the wave's own LDS tile
// (rows padded to d + 4 floats), then lane (key kk = lane % 16, slot =
// lane / 16) forms dP = dO_h . v_kk for heads slot, slot + 4, ..., stores it
// to dP[h][j] and adds P dP to its share of the chunk's row term.  The
// shares are summed over the 16 keys of a slot (xor shuffles) and over the
// waves in wave order into partD.  The waves need no workgroup barrier
// between their steps, so one wave's loads overlap another's arithmetic.
// ---------------------------------------------------------------------------
#define DEC_KW 16  // keys per wave step in k_dec_dp
template <int NL>
__global__ __launch_bounds__(256) void k_dec_dp(DecArgs a) {
  extern __shared__ float4 dyn4[];
  const int d = a.d, LD = d + 4, n4 = d / 4;
  const int g = a.H / a.KV, T = a.T, hb = min(g, 16);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* sO = reinterpret_cast<float*>(dyn4);          // [hb][d]
  float* sV = sO + hb * d + wave * DEC_KW * LD;         // this wave's [DEC_KW][d + 4]
  __shared__ float sPart[16][4];                        // [head][wave]
  const int kvh = blockIdx.x % a.KV, chunk = blockIdx.x / a.KV;  // KV heads of a chunk adjacent
  const int j0 = chunk * DEC_TB, nj = min(DEC_TB, T - j0);
  const int kk = lane & 15, slot = lane >> 4;
  for (int h0 = 0; h0 < g; h0 += 16) {
    const int hn = min(16, g - h0);
    __syncthreads();  // previous heads done with sO and sPart
    for (int i = tid; i < hn * n4; i += 256)
      reinterpret_cast<float4*>(sO)[i] =
          reinterpret_cast<const float4*>(a.dO + (size_t)(kvh * g + h0) * d)[i];
    __syncthreads();
    float pd[4] = {0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step < 2; ++step) {
      const int kb = wave * 2 * DEC_KW + step * DEC_KW;  // first key of the step in the chunk
      float4 vb[NL];
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int i = lane + 64 * u, kr = i / n4, c4 = i % n4;
        vb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < DEC_KW * n4 && kb + kr < nj)
          vb[u] = stream_load(reinterpret_cast<const float4*>(a.V) + ((size_t)(j0 + kb + kr) * a.KV + kvh) * n4 + c4);
      }
      // the wave's LDS operations run in order: the previous step's reads of
      // the tile are done before these writes, and these before the reads
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int i = lane + 64 * u, kr = i / n4, c4 = i % n4;
        if (i < DEC_KW * n4) *reinterpret_cast<float4*>(sV + kr * LD + 4 * c4) = vb[u];
      }
      __builtin_amdgcn_wave_barrier();
      float acc[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m][0] = acc[m][1] = 0.f;
      const float* vr = sV + kk * LD;
      for (int c = 0; c < d; c += 8) {
        const float4 v0 = *reinterpret_cast<const float4*>(vr + c);
        const float4 v1 = *reinterpret_cast<const float4*>(vr + c + 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int hh = slot + 4 * m;
          if (hh < hn) {
            const float4 w0 = *reinterpret_cast<const float4*>(sO + hh * d + c);
            const float4 w1 = *reinterpret_cast<const float4*>(sO + hh * d + c + 4);
            acc[m][0] = fmaf(v0.x, w0.x, fmaf(v0.y, w0.y, fmaf(v0.z, w0.z, fmaf(v0.w, w0.w, acc[m][0]))));
            acc[m][1] = fmaf(v1.x, w1.x, fmaf(v1.y, w1.y, fmaf(v1.z, w1.z, fmaf(v1.w, w1.w, acc[m][1]))));
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (kb + kk < nj) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int hh = slot + 4 * m;
          if (hh < hn) {
            const float sdp = acc[m][0] + acc[m][1];
            const size_t idx = (size_t)(kvh * g + h0 + hh) * T + j0 + kb + kk;
            a.dP[idx] = sdp;
            pd[m] = fmaf(a.P[idx], sdp, pd[m]);
          }
        }
      }
    }
    // sum over the 16 keys of each slot (every lane takes part), then the
    // slot's first lane records the wave's share of head slot + 4 m
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float x = pd[m];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o);
      const int hh = slot + 4 * m;
      if (kk == 0 && hh < hn) sPart[hh][wave] = x;
    }
    __syncthreads();
    if (tid < hn)
      a.partD[(size_t)(kvh * g + h0 + tid) * a.nch + chunk] =
          ((sPart[tid][0] + sPart[tid][1]) + sPart[tid][2]) + sPart[tid][3];
  }
}

// ---------------------------------------------------------------------------
// k_dec_kv<HB>: per (chunk, KV head), the group's heads HB at a time (HB =
// 4, 8 or 16, the smallest that holds the group or 16).  D_h for the heads
// (the partials in chunk order, a wave sum each), dS = P (dP - D) and P of
// the chunk into LDS; then thread t (t < R * d/4, R = 256 / (d/4) keys at a
// time) takes columns 4 c4 .. 4 c4 + 3 (c4 = t % (d/4)) of keys r, r + R, ...
// (r = t / (d/4)), with those columns of q_h and dO_h in registers:
// dK += scale sum_h dS q_h, dV += sum_h P dO_h, and its share of
// sum_j dS k_j per head, reduced over r (in r order) through LDS into partQ.
// ---------------------------------------------------------------------------
template <int HB>
__global__ __launch_bounds__(256) void k_dec_kv(DecArgs a) {
  constexpr int U = HB == 16 ? 2 : 4;  // keys per step with their loads in flight
  __shared__ float sS[HB][DEC_TB];   // dS of the batch's heads x the chunk's keys
  __shared__ float sPr[HB][DEC_TB];  // P of the same
  __shared__ float sD[HB];
  __shared__ float4 sRed[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvh = blockIdx.x % a.KV, chunk = blockIdx.x / a.KV;  // KV heads of a chunk adjacent
  const int g = a.H / a.KV, d = a.d, T = a.T, n4 = d / 4;
  const int j0 = chunk * DEC_TB, nj = min(DEC_TB, T - j0);
  const int R = 256 / n4, c4 = tid % n4, r = tid / n4;
  const bool active = tid < R * n4;
  for (int h0 = 0; h0 < g; h0 += HB) {
    const int hn = min(HB, g - h0);
    // D of these heads: wave w sums heads w, w+4, ... over the chunks in order
    for (int hh = wave; hh < hn; hh += 4) {
      const float* pd = a.partD + (size_t)(kvh * g + h0 + hh) * a.nch;
      float s = 0.f;
      for (int k = lane; k < a.nch; k += 64) s += pd[k];
      s = wave_sum(s);
      if (lane == 0) sD[hh] = s;
    }
    __syncthreads();
    for (int i = tid; i < hn * DEC_TB; i += 256) {
      const int hh = i / DEC_TB, jj = i % DEC_TB;
      float ds = 0.f, p = 0.f;
      if (jj < nj) {
        const size_t k = (size_t)(kvh * g + h0 + hh) * T + j0 + jj;
        p = a.P[k];
        ds = p * (a.dP[k] - sD[hh]);
      }
      sS[hh][jj] = ds;
      sPr[hh][jj] = p;
    }
    __syncthreads();
    float4 qacc[HB], qv[HB], ov[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      qacc[hh] = make_float4(0.f, 0.f, 0.f, 0.f);
      qv[hh] = ov[hh] = qacc[hh];
      if (active && hh < hn) {
        qv[hh] = reinterpret_cast<const float4*>(a.q + (size_t)(kvh * g + h0 + hh) * d)[c4];
        ov[hh] = reinterpret_cast<const float4*>(a.dO + (size_t)(kvh * g + h0 + hh) * d)[c4];
      }
    }
    if (active) {
      for (int jb = r; jb < nj; jb += U * R) {
        float4 kc[U], k0[U], v0[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // all loads of the step before any use
          const int jj = jb + u * R;
          kc[u] = k0[u] = v0[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (jj < nj) {
            const size_t off = ((size_t)(j0 + jj) * a.KV + kvh) * n4 + c4;
            kc[u] = stream_load(reinterpret_cast<const float4*>(a.K) + off);
            k0[u] = stream_load(reinterpret_cast<const float4*>(a.dK) + off);
            v0[u] = stream_load(reinterpret_cast<const float4*>(a.dV) + off);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int jj = jb + u * R;
          if (jj < nj) {
            float4 dk = make_float4(0.f, 0.f, 0.f, 0.f), dv = dk;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
              if (hh < hn) {
                const float ds = sS[hh][jj], p = sPr[hh][jj];
                dk.x = fmaf(ds, qv[hh].x, dk.x); dk.y = fmaf(ds, qv[hh].y, dk.y);
                dk.z = fmaf(ds, qv[hh].z, dk.z); dk.w = fmaf(ds, qv[hh].w, dk.w);
                dv.x = fmaf(p, ov[hh].x, dv.x); dv.y = fmaf(p, ov[hh].y, dv.y);
                dv.z = fmaf(p, ov[hh].z, dv.z); dv.w = fmaf(p, ov[hh].w, dv.w);
                qacc[hh].x = fmaf(ds, kc[u].x, qacc[hh].x); qacc[hh].y = fmaf(ds, kc[u].y, qacc[hh].y);
                qacc[hh].z = fmaf(ds, kc[u].z, qacc[hh].z); qacc[hh].w = fmaf(ds, kc[u].w, qacc[hh].w);
              }
            }
            const size_t off = ((size_t)(j0 + jj) * a.KV + kvh) * n4 + c4;
            const float sc = a.scale;
            reinterpret_cast<float4*>(a.dK)[off] =
                make_float4(k0[u].x + sc * dk.x, k0[u].y + sc * dk.y, k0[u].z + sc * dk.z, k0[u].w + sc * dk.w);
            reinterpret_cast<float4*>(a.dV)[off] =
                make_float4(v0[u].x + dv.x, v0[u].y + dv.y, v0[u].z + dv.z, v0[u].w + dv.w);
          }
        }
      }
    }
    // per head: the R threads of columns c4 add their shares, in r order
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (hh < hn) {  // the same for the whole workgroup
        sRed[tid] = active ? qacc[hh] : make_float4(0.f, 0.f, 0.f, 0.f);
        __syncthreads();
        if (tid < n4) {
          float4 t = sRed[tid];
          for (int rr = 1; rr < R; ++rr) {
            const float4 x = sRed[rr * n4 + tid];
            t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
          }
          reinterpret_cast<float4*>(a.partQ + ((size_t)chunk * a.H + kvh * g + h0 + hh) * d)[tid] = t;
        }
        __syncthreads();
      }
    }
  }
}

// k_dec_dq: dq[h][c] += scale * sum over chunks of partQ[chunk][h][c].  A
// workgroup of 16 waves takes 64 consecutive (h, c); wave w sums chunks
// w, w + 16, ... in order, and the 16 wave sums are added in wave order.
#define DEC_DQ_WAVES 16
__global__ __launch_bounds__(64 * DEC_DQ_WAVES) void k_dec_dq(DecArgs a) {
  __shared__ float sW[DEC_DQ_WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long n = (long long)a.H * a.d;
  const long long i = (long long)blockIdx.x * 64 + lane;
  float s = 0.f;
  if (i < n) {
#pragma unroll 4
    for (int k = wave; k < a.nch; k += DEC_DQ_WAVES) s += a.partQ[(size_t)k * n + i];
  }
  sW[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && i < n) {
    float t = sW[0][lane];
#pragma unroll
    for (int w = 1; w < DEC_DQ_WAVES; ++w) t += sW[w][lane];
    a.dq[i] += a.scale * t;
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

extern "C" attn_status_t attn_bwd_decode(const float* q, const float* K, const float* V,
                                         const float* P, const float* dO, float* dq, float* dK,
                                         float* dV, int history_len, int n_heads, int n_kv_heads,
                                         int head_dim, float scale, void* stream) {
  clear_error();
  // an empty history has no K, V, P, dK, dV (a framework may pass NULL for them)
  if (!q || !dO || !dq || (history_len != 0 && (!K || !V || !P || !dK || !dV)))
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  attn_status_t rc = check_common(history_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {q, K, V, P, dO, dq, dK, dV};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (history_len == 0) return ATTN_OK;

  const int nch = (history_len + DEC_TB - 1) / DEC_TB;
  const size_t off_dP = 0;
  const size_t off_pD = align256((size_t)n_heads * history_len * 4);
  const size_t off_pQ = off_pD + align256((size_t)n_heads * nch * 4);
  const size_t bytes = off_pQ + align256((size_t)nch * n_heads * head_dim * 4);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipMemPool_t pool;
  rc = device_pool(&pool);
  if (rc != ATTN_OK) return rc;
  void* ws = nullptr;
  rc = hip_check(hipMallocFromPoolAsync(&ws, bytes, pool, st), "hipMallocFromPoolAsync(workspace)");
  if (rc != ATTN_OK) return rc;
  char* w = static_cast<char*>(ws);

  DecArgs a;
  a.q = q; a.K = K; a.V = V; a.P = P; a.dO = dO;
  a.dq = dq; a.dK = dK; a.dV = dV;
  a.dP = reinterpret_cast<float*>(w + off_dP);
  a.partD = reinterpret_cast<float*>(w + off_pD);
  a.partQ = reinterpret_cast<float*>(w + off_pQ);
  a.T = history_len; a.H = n_heads; a.KV = n_kv_heads; a.d = head_dim; a.nch = nch;
  a.scale = scale;

  rc = profile_mark(st, true);
  if (rc == ATTN_OK) {
    const int hb = std::min(n_heads / n_kv_heads, 16);
    const size_t lds = ((size_t)hb * head_dim + 4 * DEC_KW * (head_dim + 4)) * 4;  // 36 KB at d = 128, 4 heads
    if (head_dim <= 64)
      hipLaunchKernelGGL(k_dec_dp<4>, dim3(nch * n_kv_heads), dim3(256), lds, st, a);
    else if (head_dim <= 128)
      hipLaunchKernelGGL(k_dec_dp<8>, dim3(nch * n_kv_heads), dim3(256), lds, st, a);
    else
      hipLaunchKernelGGL(k_dec_dp<16>, dim3(nch * n_kv_heads), dim3(256), lds, st, a);
    rc = hip_check(hipGetLastError(), "launching k_dec_dp");
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc == ATTN_OK) {
    const int g = n_heads / n_kv_heads;
    if (g <= 4)
      hipLaunchKernelGGL(k_dec_kv<4>, dim3(nch * n_kv_heads), dim3(256), 0, st, a);
    else if (g <= 8)
      hipLaunchKernelGGL(k_dec_kv<8>, dim3(nch * n_kv_heads), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_dec_kv<16>, dim3(nch * n_kv_heads), dim3(256), 0, st, a);
    rc = hip_check(hipGetLastError(), "launching k_dec_kv");
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc == ATTN_OK) {
    const int blocks = (int)(((long long)n_heads * head_dim + 63) / 64);
    hipLaunchKernelGGL(k_dec_dq, dim3(blocks), dim3(64 * DEC_DQ_WAVES), 0, st, a);
    rc = hip_check(hipGetLastError(), "launching k_dec_dq");
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  attn_status_t rc2 = hip_check(hipFreeAsync(ws, st), "hipFreeAsync(workspace)");
  return rc != ATTN_OK ? rc : rc2;
}
