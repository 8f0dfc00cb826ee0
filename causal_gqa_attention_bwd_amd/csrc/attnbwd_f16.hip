// attnbwd_f16.hip -- the attention backward with 16-bit matrix-core operands
// (attn_bwd_f16): the gradients of page "llm.istanbul --
// 10_backward_attention.wgsl" (kernel attention_backward: P, dP, D, dS, then
// dV = P^T dO, dK = dS^T Q, dQ = dS K, all +=), with every product operand --
// Q, K, V, dO, the probabilities P and the score gradients scale*dS -- rounded
// to fp16 (round to nearest even) and every sum accumulated in fp32.  Inputs,
// outputs, LSE, the row term D, the exponent and the masks stay fp32.  The
// pages compute in fp32 throughout; this is the reduced-precision variant of
// the same sums, at 16 times the fp32 matrix rate of the hardware.
//
// Per call:
//   k_prep    per 32-row query block seg min / max and tile slots (shared
//             with attn_bwd).
//   k_cvt16   fp16 copies of Q, dO, K, V as head-major row tiles [head][Sp][DP]
//             (Sp = S rounded up to 128, DP = head_dim rounded up to a tile
//             width; padding is zero).
//   D         k_rowdot (D = dO . O) when the forward output is given, else
//             k_q16<D only>: S^T and dP^T of every visible pair, D = sum P dP.
//   k_kv16    key-major, one workgroup per (128-key tile, KV head, head
//             split, column part), owns its dK / dV rows and sums its heads:
//             S = Q K^T, dP = dO V^T, P, dS, dV += P^T dO, dK += dS^T Q.  4
//             products per visible pair; stores each dS/scale tile in fp16
//             for the dQ pass.  k_kv16r: the same with each key block's work
//             split over two waves by role (up to 128 columns).
//   k_dqs16   query-major, one workgroup per (128-query tile, head): dQ +=
//             (dS/scale) K from the stored tiles.  1 product per visible pair.
//   k_q16     (only when the dS tiles do not fit the scratch limit or the
//             pool) the same dQ, forming S^T, dP^T and dS again: 3 products.
// Executed products per visible pair: 5 with the forward output, 7 without
// (the page's method credits 5).
//
// MFMA v_mfma_f32_32x32x16_f16 (C[32x32] += A[32x16] B[16x32]), lane layout
// checked on the device: lane l supplies A[l%32][8(l/32) + j] and
// B[8(l/32) + j][l%32] for j = 0..7 (16 bytes each) and holds C like the fp32
// product (register r: row crow(r, l/32), column l%32).  Registers 8s..8s+7 of
// an accumulator tile, rounded to fp16, are therefore the A operand of a
// product that contracts over the tile's rows, taken in the row order
// crow(8s + j, hf).  The matching B operand (those rows, one column per lane)
// comes from the staged row tile through two transposing LDS loads
// (tr_operand below), so no transposed copy of any tensor is made.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// out_rsrc for an address and size that every lane of the wave holds, taken
// from lane 0: the compiler then keeps the descriptor in scalar registers
// (else, not proving the values uniform, it wraps every access in a loop
// over the distinct descriptors of the wave and waits for each access)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const float* p, uint32_t bytes) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return out_rsrc((void*)(((uint64_t)hi << 32) | lo), (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes));
}

__device__ __forceinline__ f32x16 mfma16(const h8& a, const h8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Registers 8s .. 8s+7 of accumulator tile c, rounded to fp16 (nearest even).
__device__ __forceinline__ h8 pack8(const f32x16& c, int s) {
  f32x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = c[8 * s + j];
  return __builtin_convertvector(v, h8);
}

// The B operand of a 32x32x16 product -- lane l supplies B[8 (l/32) + j]
// [l%32], j = 0..7 -- read straight from a row-major Tile16 (its rows are
// the contraction index, 8 columns per 16-byte chunk) by two transposing LDS
// loads (ds_read_b64_tr_b16).  Within each group of 16 lanes such a load
// hands lane i, as element j, the (i mod 4)-th 16-bit value of the 8 bytes
// that lane 4j + i/4 of the group addressed (checked on the device).  So
// lane L = 4a + b of group G addresses row r + a, columns n0 + 16 (G % 2) +
// 4b .. + 3, and receives column n0 + 16 (G % 2) + L = n0 + l%32 of rows
// r .. r + 3.  The caller gives the first tile row of each load (row_c0 for
// j = 0..3, row_c1 for j = 4..7), for the rows of its lane's half-wave.
typedef short s4v __attribute__((__vector_size__(8)));
typedef short s8v __attribute__((ext_vector_type(8)));
template <class T>
__device__ __forceinline__ h8 tr_operand(const char* tile, int row_c0, int row_c1, int n0, int lane) {
  const int L = lane & 15, G = lane >> 4;
  const int col = n0 + 16 * (G & 1) + 4 * (L & 3);
  const uint32_t sub = (uint32_t)(col & 7) * 2u;  // 0 or 8 bytes into the 16-byte chunk
  const char* p0 = tile + T::at(row_c0 + (L >> 2), col >> 3) + sub;
  const char* p1 = tile + T::at(row_c1 + (L >> 2), col >> 3) + sub;
  const s4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)p0);
  const s4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)p1);
  const s8v v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(h8, v);
}

// ---------------------------------------------------------------------------
// fp16 tiles in LDS: ROWS x CH chunks of 16 bytes, unpadded; chunk c of row r
// sits at chunk r*CH + (c ^ swz(r)).  Two reads meet these tiles: 16-byte
// reads of 8 (and 16) consecutive rows at one chunk (the row operands), and
// the transposing 8-byte reads of 4 consecutive rows at 4 adjacent chunks
// (tr_operand; 2 chunks per 16 lanes).  The swizzle, a linear map of the row's
// low four bits (b0..b3), was found by exhaustive search to make both hit
// distinct banks, counting 64 banks (16 chunk slots) and 32 (8 chunk slots),
// for every CH used here (4, 8, 12, 16, 24, 32), and keeps c ^ swz(r) < CH.
// ---------------------------------------------------------------------------
template <int CH>
__device__ __forceinline__ int swz(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
  if constexpr (CH % 8 != 0) return (b1 << 1) ^ b2 ^ (b3 << 1);
  else if constexpr (CH % 16 != 0) return (b0 << 1) ^ (b1 << 2) ^ b2 ^ (b3 << 1);
  else return (b0 << 2) ^ (b1 * 10) ^ b2 ^ (b3 << 1);
}

template <int ROWS, int CH>
struct Tile16 {
  static constexpr int CHUNKS = ROWS * CH;
  // wave-wide 1 KiB loads per tile, a multiple of 4 so that every wave issues
  // the same number (the surplus loads deposit zeros past the tile's chunks)
  static constexpr int NCH = (CHUNKS + 255) / 256 * 4;
  static constexpr int BYTES = NCH * 1024;
  static constexpr int CPW = NCH / 4;              // loads per wave
  // LDS byte offset of chunk c of row r
  __device__ static __forceinline__ uint32_t at(int r, int c) {
    return (uint32_t)(r * CH + (c ^ swz<CH>(r))) * 16u;
  }
};

// Per-lane global byte offsets of the chunks this wave loads into a Tile16
// whose rows are `gstride` bytes apart in memory: physical chunk p of the tile
// takes logical chunk (p % CH) ^ swz(p / CH) of row p / CH.
template <int ROWS, int CH>
struct Loader16 {
  using T = Tile16<ROWS, CH>;
  uint32_t off[T::CPW];
  __device__ __forceinline__ void init(uint32_t gstride, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) {
      const int p = (wave + 4 * i) * 64 + lane;
      const int r = p / CH, c = (p % CH) ^ swz<CH>(p / CH);
      off[i] = p < T::CHUNKS ? (uint32_t)r * gstride + (uint32_t)c * 16u : ATTN_BUF_OOB;
    }
  }
  __device__ __forceinline__ void load(const i32x4& rs, uint32_t lds_byte, int wave) const {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) dma16(rs, off[i], lds_byte + (wave + 4 * i) * 1024);
  }
};

// Wait until at most N of this wave's vector-memory operations (its
// direct-to-LDS loads among them) are outstanding; loads retire in issue
// order, so everything issued before the last N has landed.  Other counters
// are left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct F16Args {
  const _Float16 *Qh, *dOh, *Kh, *Vh;  // [heads][Sp][DP] row tiles
  const float* LSE;                    // [S, H]
  const uint32_t* seg;                 // [S], NULL = all zeros
  float *dQ, *dK, *dV;
  float* D;                            // [S, H] row term
  const uint32_t* blk_min;             // [ceil(S/32)] min seg per 32-row query block
  const uint32_t* blk_max;             // [ceil(S/32)] max seg per 32-row query block
  const float* LSE2;                   // [S, H] LSE * log2(e) (k_cvt16)
  const long long* slot_off;           // [ceil(S/32) + 1] first tile slot of each query block
  // blk_min, blk_max and slot_off as one buffer from blk_min (the step's
  // metadata is staged with one load): its size and the byte offsets of
  // blk_max and slot_off in it
  uint32_t meta_bytes, meta_max, meta_slot;
  // the stored dS/scale tiles (fp16, 2 KiB per (slot, head): keys as rows,
  // see ds_tile_row), written by the key-major pass and read by k_dqs16; NULL
  // when they do not fit the scratch limit (k_q16 then recomputes dS)
  _Float16* dS;
  int S, Sp, H, KV, d;
  float scale;
  int pair;                            // 1: block p serves tiles p and n-1-p (plain causal)
  int splits;                          // k_kv16: workgroups sharing one key tile's heads
  int kv_work;                         // k_kv16: (key tile, KV head, split) triples
  float* part;                         // [2 * splits][S, KV, d] partial dK, dV (splits > 1)
  int rope;                            // 1: dQ, dK rotated back by RoPE in the write-back
  int rope_pos;                        // position of row 0 (the page's pos_offset)
  double rope_base;                    // frequency base
};

// Where lane `lane` of the loading wave takes query block qb's staged
// metadata from (one 4-byte load per lane into 256 bytes of the stage; lanes
// 4.. deposit zeros): lane 0 the block's largest document start (0 without a
// seg), lane 1 its smallest, lanes 2 and 3 its first tile slot (64-bit).
__device__ __forceinline__ uint32_t meta_off(const F16Args& a, int qb, int lane) {
  // every candidate formed, then selected (no divergent branch per lane)
  const uint32_t q4 = 4u * (uint32_t)qb;
  const uint32_t o_max = a.meta_max + q4, o_slot = a.meta_slot + 2u * q4 + 4u * (uint32_t)(lane & 1);
  uint32_t off = lane < 4 ? o_slot : ATTN_BUF_OOB;
  off = lane == 1 ? q4 : off;
  return lane == 0 ? o_max : off;
}

// Stored dS/scale tiles.  The tile of (query block qb, key block kb, head h)
// is tile slot slot_off[qb] + kb - blk_min[qb]/32 (the slots of k_prep: the
// key blocks from the block's first document start to the diagonal), 2 KiB
// at ((slot * H) + h) * 2 KiB.  A key-major lane l (key l%32, half hf =
// l/32) holds dS/scale of queries crow(8s + j, hf), s = 0, 1, j = 0..7, as
// the two packed operands of its dK product, and writes operand s as the 16
// bytes at 1024 s + 16 l: each store is 1 KiB of consecutive bytes.  Read as
// 32 key rows of 32 values, column c = 16 hf + 8 s + j of key row r is the
// value at 1024 s + 16 (r + 32 hf) + 2 j, and it holds query ds_query(c) of
// the block.
__device__ __forceinline__ int ds_query(int c) {
  return 16 * ((c >> 3) & 1) + 8 * ((c >> 2) & 1) + 4 * (c >> 4) + (c & 3);
}

// The dS/scale tile of key block kbk, head `head`, for the query block whose
// staged metadata `m` is (the 16 bytes meta_off places: largest and smallest
// document start, first slot), or NULL when the key block lies before the
// block's first document start (the tile has no slot, and its dS is zero).
__device__ __forceinline__ _Float16* ds_tile(const F16Args& a, const uint4& m, int kbk, int head) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)m.y) / 32u;
  if ((uint32_t)kbk < lo) return nullptr;
  const long long slot = (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)m.w) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((int)m.z));
  return a.dS + ((size_t)(slot + kbk - (long long)lo) * a.H + head) * 1024;
}

// Write a tile's two operands held by lane `lane` (see ds_query) to t.
__device__ __forceinline__ void ds_write(_Float16* t, int lane, const h8& d0, const h8& d1) {
  const auto r = out_rsrc(t, 2048u);
  // non-temporal (read once, by another kernel)
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, d0), r, 16u * lane, 0, ATTN_CPOL_NT);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, d1), r, 16u * lane + 1024u, 0,
                                         ATTN_CPOL_NT);
}

struct CvtArgs {
  const float *Q, *dO, *K, *V;
  _Float16 *Qh, *dOh, *Kh, *Vh;
  const float* LSE;                    // [S, H]
  float* LSE2;                         // [S, H] LSE * log2(e), for k_kv16
  int S, Sp, H, KV, d;
};

// ---------------------------------------------------------------------------
// k_cvt16: one workgroup per (32-row block, head) of one tensor; blocks
// [0, nb*H) convert Q, then dO, then K (nb*KV), then V.  Rows past S and
// columns past head_dim become zeros.  The Q blocks also write their rows'
// LSE * log2(e), the exponent offset k_kv16 stages per step.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void k_cvt16(CvtArgs a) {
  const int nb = a.Sp / 32;
  const long long nq = (long long)nb * a.H, nk = (long long)nb * a.KV;
  long long b = blockIdx.x;
  int which;
  if (b < nq) which = 0;
  else if (b < 2 * nq) { which = 1; b -= nq; }
  else if (b < 2 * nq + nk) { which = 2; b -= 2 * nq; }
  else { which = 3; b -= 2 * nq + nk; }
  const int heads = which < 2 ? a.H : a.KV;
  const int head = (int)(b % heads);
  const int r0 = (int)(b / heads) * 32;
  const float* src = which == 0 ? a.Q : which == 1 ? a.dO : which == 2 ? a.K : a.V;
  _Float16* dst = which == 0 ? a.Qh : which == 1 ? a.dOh : which == 2 ? a.Kh : a.Vh;
  const size_t stride = (size_t)heads * a.d;
  const int nrows = max(0, min(32, a.S - r0));
  // chunks of 4 columns: 16-byte reads, 8-byte writes (head_dim is a multiple
  // of 16).  Every read of the thread is issued before its first write, so
  // the reads overlap instead of each waiting behind the previous write; a
  // chunk past S or head_dim reads zeros from beyond the buffer range.
  constexpr int PER = 32 * (DP / 4) / 256;  // chunks per thread
  static_assert(32 * (DP / 4) % 256 == 0, "whole chunks per thread");
  const auto rs = wave_rsrc(src + (size_t)r0 * stride + (size_t)head * a.d,
                            nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * stride + a.d) * 4) : 0u);
  f32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + 256 * k, r = i / (DP / 4), c = 4 * (i % (DP / 4));
    const uint32_t off = (r < nrows && c < a.d) ? (uint32_t)(((size_t)r * stride + c) * 4) : ATTN_BUF_OOB;
    v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + 256 * k, r = i / (DP / 4), c = 4 * (i % (DP / 4));
    *reinterpret_cast<h4*>(dst + ((size_t)head * a.Sp + r0 + r) * DP + c) = __builtin_convertvector(v[k], h4);
  }
  if (which == 0 && threadIdx.x < 32 && r0 + (int)threadIdx.x < a.S) {
    const size_t i = (size_t)(r0 + threadIdx.x) * a.H + head;
    a.LSE2[i] = a.LSE[i] * ATTN_LOG2E;
  }
}

// Column pair (2p, 2p + 1) = (x0, x1) of a row at position pos turned back by
// the RoPE rotation, both columns from one sincos: the arithmetic of
// rope_back for each column.
__device__ __forceinline__ f32x2 rope_back_pair(float x0, float x1, long long pos, double freq) {
  double sn, cs;
  sincos((double)pos * freq, &sn, &cs);
  return f32x2{(float)((double)x0 * cs + (double)x1 * sn), (float)(-(double)x0 * sn + (double)x1 * cs)};
}

// ---------------------------------------------------------------------------
// dQ += scale * acc for one wave's 32 query rows r0 + rowof(r) (register r of
// each 32-column output tile o), or with RoPE dQ = R^T (dQ + scale * acc), the
// pair partner column in lane l ^ 1, through a buffer over the wave's rows:
// rows past S and columns past head_dim read zero and drop their stores, so
// every lane reaches the partner exchange.
// ---------------------------------------------------------------------------
template <int NO, bool ROPE, bool BUF, class RowOf>
__device__ __forceinline__ void dq_writeback(const F16Args& a, const f32x16 (&acc)[NO], int h, int r0,
                                             int hf, int l32, RowOf rowof) {
  const size_t qstride = (size_t)a.H * a.d;
  if constexpr (!ROPE && !BUF) {
    // (a load, add and store per element behind a branch: the k_q16 form,
    // whose registers do not hold the buffer form's offsets)
    float* dQh = a.dQ + (size_t)h * a.d;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      const int col = 32 * o + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + rowof(r);
        if (row < a.S && col < a.d) dQh[(size_t)row * qstride + col] += a.scale * acc[o][r];
      }
    }
  } else if constexpr (!ROPE) {
    // through a buffer over the wave's rows, no branch per element: every
    // load of an output tile is issued before its adds and stores
    const int nrows = max(0, min(32, a.S - r0));
    const auto rq = out_rsrc(a.dQ + (size_t)h * a.d + (size_t)r0 * qstride,
                             nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * qstride + a.d) * 4) : 0u);
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      const int col = 32 * o + l32;
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 8) {
        uint32_t off[8];
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int rr = rowof(r0 + r);
          off[r] = (rr < nrows && col < a.d) ? (uint32_t)(((size_t)rr * qstride + col) * 4) : ATTN_BUF_OOB;
          v[r] = buf_ld(rq, off[r]);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) buf_st(rq, off[r], v[r] + a.scale * acc[o][r0 + r]);
        __builtin_amdgcn_sched_barrier(0);  // eight rows at a time
      }
    }
  } else {
    const int nrows = max(0, min(32, a.S - r0));
    const auto rq = out_rsrc(a.dQ + (size_t)h * a.d + (size_t)r0 * qstride,
                             nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * qstride + a.d) * 4) : 0u);
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      const int col = 32 * o + l32;
      const double fq = rope_freq(col, a.d, a.rope_base);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = rowof(r);
        const uint32_t off = (rr < nrows && col < a.d) ? (uint32_t)(((size_t)rr * qstride + col) * 4)
                                                       : ATTN_BUF_OOB;
        const float v = buf_ld(rq, off) + a.scale * acc[o][r];
        buf_st(rq, off, rope_back(v, __shfl_xor(v, 1), col, (long long)r0 + rr + a.rope_pos, fq));
      }
      __builtin_amdgcn_sched_barrier(0);  // one output tile at a time
    }
  }
}

// ---------------------------------------------------------------------------
// k_q16: query-major, one workgroup per (128-query tile, head).  Wave w owns
// queries i0 + 32w + l%32 and keeps their Q and dO rows in registers as the B
// operands of S^T = K Q^T and dP^T = V dO^T; 32-key blocks of K, V (row
// tiles) and K^T stream through an LDS ring of NBUF stages (NBUF - 1 blocks
// in flight), shared by the four waves.  The score tiles hold key crow(r, hf)
// of query l%32, so each lane's LSE, D and seg are one value.
//   DONLY: D[q] = sum_j P dP (the row term, for the key-major pass).
//   else:  dQ += scale (dS/scale) K with dS/scale = P (dP - D), A operand
//          straight from the dS registers, B from the K row tile by
//          transposing loads; the accumulators stay in AGPRs.
// A block whose every pair is visible (keys at or before every query of the
// wave, at or after every row's document start, every row inside S) skips
// the per-element mask; the wave's largest document start comes from k_prep.
// ---------------------------------------------------------------------------
template <int DP, bool DONLY>
struct QGeom {
  using RT = Tile16<32, DP / 8>;
  static constexpr int STAGE = 2 * RT::BYTES;
  // two workgroups per CU up to 128 columns; above, one in dQ mode, and two
  // for the row term (fewer registers) with a shallower ring (S=16384, d=256:
  // 0.77 -> 0.60 ms; three per CU up to 128 columns gained nothing)
  static constexpr int BUDGET = DP <= 128 ? 72 * 1024 : DONLY ? 72 * 1024 : 150 * 1024;
  static constexpr int WAVES_PER_SIMD = DP <= 128 || DONLY ? 2 : 1;
  static constexpr int NBUF = 4 * STAGE <= BUDGET ? 4 : 3 * STAGE <= BUDGET ? 3 : 2;
  static constexpr int LPS = 2 * RT::CPW;  // loads per wave per block
  static_assert((NBUF - 2) * LPS < 64, "loads in flight fit vmcnt");
};

template <int DP, bool DONLY, bool ROPE>
__global__ __launch_bounds__(256, (QGeom<DP, DONLY>::WAVES_PER_SIMD)) void k_q16(F16Args a) {
  using G = QGeom<DP, DONLY>;
  using RT = typename G::RT;
  constexpr int NT = DP / 16;  // k-steps of the d-contractions
  constexpr int NO = DP / 32;  // 32-column output tiles
  constexpr int NBUF = G::NBUF, STAGE = G::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H;
  const int g = H / a.KV;
  const int qt_hi = (S - 1) / 128;
  const float sc2 = a.scale * ATTN_LOG2E;
  const uint32_t smem0 = lds_addr(smem);
  Loader16<32, DP / 8> ldr;
  ldr.init(DP * 2, wave, lane);

  auto tile = [&](const int qt) __attribute__((always_inline)) {
    const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
    const int i0 = qt * 128;
    const int q = i0 + 32 * wave + l32;  // < Sp: the copies hold zero rows up to Sp
    const bool q_ok = q < S;
    h8 qreg[NT], oreg[NT];
    const _Float16* qrow = a.Qh + ((size_t)h * a.Sp + q) * DP + 8 * hf;
    const _Float16* orow = a.dOh + ((size_t)h * a.Sp + q) * DP + 8 * hf;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qreg[t] = *reinterpret_cast<const h8*>(qrow + 16 * t);
      oreg[t] = *reinterpret_cast<const h8*>(orow + 16 * t);
    }
    const float lse2 = q_ok ? a.LSE[(size_t)q * H + h] * ATTN_LOG2E : 0.f;
    const uint32_t sq = !q_ok ? 0xffffffffu : (a.seg ? a.seg[q] : 0u);
    float Dq = 0.f;
    if constexpr (!DONLY) Dq = q_ok ? a.D[(size_t)q * H + h] : 0.f;

    // key blocks: from the smallest document start of the tile to the diagonal
    const int nblk = (S + 31) / 32;
    const int qb = (i0 >> 5) + wave;
    const uint32_t lo = qb < nblk ? a.blk_min[qb] : 0xffffffffu;
    // the largest document start of this wave's rows, and whether all 32 exist
    const uint32_t wmx = (a.seg && qb < nblk) ? a.blk_max[qb] : 0u;
    const int q_first = i0 + 32 * wave;
    const bool rows_in = q_first + 31 < S;
    if (lane == 0) sMin[wave] = lo;
    // the register loads above land here, where the compiler sees it (not
    // inside the block loop, on a counter that also counts the ring's loads)
    wait_vm<0>();
    __syncthreads();
    const uint32_t lo_all = min(min(sMin[0], sMin[1]), min(sMin[2], sMin[3]));
    const int kb_last = min(i0 + 127, S - 1) / 32;
    const int kb_first = (int)min(lo_all / 32u, (uint32_t)kb_last + 1u);
    const int n = kb_last - kb_first + 1;  // blocks of the tile (0: none)
    // this wave's key blocks (a wave past S has lo = ~0 and sees none)
    const int w_lo = (int)min(lo / 32u, 0x7fffffffu);
    const int w_hi = min(i0 + 32 * wave + 31, S - 1) / 32;

    auto issue = [&](int kb, int buf) {
      const uint32_t st = smem0 + (uint32_t)(buf * STAGE);
      const size_t roff = ((size_t)kvh * a.Sp + (size_t)kb * 32) * DP;
      ldr.load(buf_rsrc(a.Kh + roff, 32 * DP * 2), st, wave);
      ldr.load(buf_rsrc(a.Vh + roff, 32 * DP * 2), st + RT::BYTES, wave);
    };

    f32x16 acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      acc[o] = zero16();
      if constexpr (!DONLY) asm volatile("" : "+a"(acc[o]));
    }
    float Dacc = 0.f;

    auto compute = [&](int kb, int buf) {
      if (kb < w_lo || kb > w_hi) return;
      const char* st = smem + buf * STAGE;
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const h8 ka = *reinterpret_cast<const h8*>(st + RT::at(l32, 2 * t + hf));
        const h8 va = *reinterpret_cast<const h8*>(st + RT::BYTES + RT::at(l32, 2 * t + hf));
        s = mfma16(ka, qreg[t], s);
        dp = mfma16(va, oreg[t], dp);
      }
      // every pair visible: the block's keys at or before every query of the
      // wave, at or after every row's document start, and all rows inside S
      const bool full = rows_in & (kb * 32 + 31 <= q_first) & (wmx <= (uint32_t)(kb * 32));
      // P; the row term D += P dP, or dS/scale = P (dP - D) (the scale goes
      // onto dQ at the end)
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse2));
          if constexpr (DONLY) Dacc = fmaf(p, dp[r], Dacc);
          else s[r] = p * (dp[r] - Dq);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + crow(r, hf);
          const bool vis = (key <= q) & ((uint32_t)key >= sq);
          const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse2));
          const float p = vis ? e : 0.f;
          if constexpr (DONLY) Dacc = fmaf(p, dp[r], Dacc);
          else s[r] = p * (dp[r] - Dq);
        }
      }
      if constexpr (!DONLY) {
        // B operands from the K row tile (transposing loads): the k order of
        // a0 is keys crow(j, hf), j = 0..7 (rows 4 hf .. 4 hf + 3, then 8 +
        // 4 hf ..), of a1 the same plus 16
        const h8 a0 = pack8(s, 0), a1 = pack8(s, 1);
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          const h8 k0 = tr_operand<RT>(st, 4 * hf, 8 + 4 * hf, 32 * o, lane);
          const h8 k1 = tr_operand<RT>(st, 16 + 4 * hf, 24 + 4 * hf, 32 * o, lane);
          acc[o] = mfma16(a0, k0, acc[o]);
          acc[o] = mfma16(a1, k1, acc[o]);
          // the next tile's operand loads stay behind this point: hoisting
          // them all would not fit two waves' registers per SIMD
          asm volatile("" : "+a"(acc[o])::"memory");
        }
      }
    };

    // the ring: blocks i .. i + NBUF - 2 issued ahead of the compute of block i
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < n) issue(kb_first + k, k);
    for (int i = 0; i < n; ++i) {
      // this wave's loads of block i have landed once at most those of the
      // later issued blocks are outstanding
      const int ahead = min(NBUF - 2, n - 1 - i);
      if constexpr (NBUF >= 4) {
        if (ahead >= 2) wait_vm<2 * G::LPS>();
        else if (ahead == 1) wait_vm<G::LPS>();
        else wait_vm<0>();
      } else if constexpr (NBUF == 3) {
        if (ahead >= 1) wait_vm<G::LPS>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
      // every wave: block i resident and done with block i - 1 (whose buffer
      // the next issue refills)
      asm volatile("s_barrier" ::: "memory");
      if (i + NBUF - 1 < n) issue(kb_first + i + NBUF - 1, (i + NBUF - 1) % NBUF);
      compute(kb_first + i, i % NBUF);
    }

    if constexpr (DONLY) {
      const float Dt = Dacc + __shfl_xor(Dacc, 32);  // the half-waves saw disjoint keys
      if (q_ok && hf == 0) a.D[(size_t)q * H + h] = Dt;
    } else {
      dq_writeback<NO, ROPE, false>(a, acc, h, i0 + 32 * wave, hf, l32, [&](int r) { return crow(r, hf); });
    }
  };
  // longest rows first; paired: then the mirror tile
  const int first = qt_hi - (int)(blockIdx.x / H);
  const int second = mirror_tile(first, qt_hi + 1, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // every wave done with the ring and sMin of the first tile
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_dqs16: dQ from the stored dS/scale tiles (written by the key-major pass),
// so that dS is not formed a second time.  Query-major, one workgroup per
// (128-query tile, head), as k_q16; wave w owns query block i0/32 + w.  Per
// key block of the tile, the K row tile (all four waves load a share) and
// each wave's own dS tile of that key block stream through an LDS ring of
// NBUF stages; the wave's product dQ += (dS/scale) K takes both operands from
// transposing loads: the A operand from the dS tile (keys are its rows, the
// lane's query its column), the B operand from the K row tile.  The dS
// tile's columns hold the block's queries in the order ds_query gives, so
// accumulator row m is query ds_query(m).  One product per visible pair; the
// dS tiles (2 bytes per visible pair and head) are the kernel's HBM traffic.
// ---------------------------------------------------------------------------
template <int DP, bool ROPE>
struct DqsGeom {
  using KT = Tile16<32, DP / 8>;     // K row tile of a key block
  using DT = Tile16<32, 4>;          // one wave's dS tile: 32 keys x 32 queries
  static constexpr int OFF_DS = KT::BYTES;
  static constexpr int STAGE = KT::BYTES + 4 * 2048;
  // two workgroups per CU with a 4-stage ring; one with RoPE above 128
  // columns (the rotation's registers do not fit two waves per SIMD there).
  // Measured at S=4096, d=128: three per CU with 3 stages the same, four with
  // 2 stages and one with 9 slower (0.187, 0.185, 0.203, 0.341 ms): the
  // kernel wants waves, not a deeper ring
  static constexpr int WG_PER_CU = ROPE && DP > 128 ? 1 : 2;
  static constexpr int BUDGET = (WG_PER_CU == 1 ? 150 : 72) * 1024;
  static constexpr int NBUF = BUDGET / STAGE >= 4 ? 4 : BUDGET / STAGE;
  static constexpr int LPS = KT::CPW + 2;  // loads per wave per block
  // output tiles whose K operands are read ahead of their products at once
  // (above 128 columns the accumulators leave room for two)
  static constexpr int GO = DP > 128 ? 2 : 4;
  static_assert(NBUF >= 2, "a stage in flight");
  static_assert((NBUF - 2) * LPS < 64, "loads in flight fit vmcnt");
};

// Wait until this wave's loads of the block `ahead` blocks before the last
// issued one have landed: at most ahead * LPS loads (those of the later
// blocks) outstanding; ahead is at most MAXA.
template <int MAXA, int LPS>
__device__ __forceinline__ void wait_blocks(int ahead) {
  if constexpr (MAXA <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= MAXA) wait_vm<MAXA * LPS>();
    else wait_blocks<MAXA - 1, LPS>(ahead);
  }
}

template <int DP, bool ROPE>
__global__ __launch_bounds__(256, (DqsGeom<DP, ROPE>::WG_PER_CU)) void k_dqs16(F16Args a) {
  using G = DqsGeom<DP, ROPE>;
  using KT = typename G::KT;
  using DT = typename G::DT;
  constexpr int NO = DP / 32, NBUF = G::NBUF, STAGE = G::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];
  __shared__ uint32_t sMin[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H;
  const int g = H / a.KV;
  const int nblk = (S + 31) / 32;
  const int qt_hi = (S - 1) / 128;
  const uint32_t smem0 = lds_addr(smem);
  Loader16<32, DP / 8> ldr;
  ldr.init(DP * 2, wave, lane);
  // this lane's two chunks of its wave's dS tile: physical chunk p = lane +
  // 64 i of the 32 x 4 chunk tile takes chunk c = (p % 4) ^ swz(p / 4) of key
  // row r = p / 4, i.e. columns 8c .. 8c + 7, stored at 1024 (c % 2) + 16 (r
  // + 32 (c / 2))
  uint32_t doff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i, r = p >> 2, c = (p & 3) ^ swz<4>(r);
    doff[i] = (uint32_t)(1024 * (c & 1) + 16 * (r + 32 * (c >> 1)));
  }

  auto tile = [&](const int qt) __attribute__((always_inline)) {
    const int h = xcd_head((int)(blockIdx.x % H), H), kvh = h / g;
    const int i0 = qt * 128;
    const int qb = (i0 >> 5) + wave;
    const uint32_t lo = qb < nblk ? a.blk_min[qb] : 0xffffffffu;
    const long long slot0 = qb < nblk ? a.slot_off[qb] : 0;
    if (lane == 0) sMin[wave] = lo;
    __syncthreads();
    const uint32_t lo_all = min(min(sMin[0], sMin[1]), min(sMin[2], sMin[3]));
    const int kb_last = min(i0 + 127, S - 1) / 32;
    const int kb_first = (int)min(lo_all / 32u, (uint32_t)kb_last + 1u);
    const int n = kb_last - kb_first + 1;  // blocks of the tile (0: none)
    // this wave's key blocks, the slots of its query block (a wave past S
    // has lo = ~0 and sees none)
    const int w_lo = (int)min(lo / 32u, 0x7fffffffu);
    const int w_hi = min(i0 + 32 * wave + 31, S - 1) / 32;

    auto issue = [&](int kb, int buf) {
      const uint32_t st = smem0 + (uint32_t)(buf * STAGE);
      ldr.load(buf_rsrc(a.Kh + ((size_t)kvh * a.Sp + (size_t)kb * 32) * DP, 32 * DP * 2), st, wave);
      // the wave's dS tile (zeros, without a memory access, when the block
      // has no slot for this wave's queries)
      const bool vis = kb >= w_lo && kb <= w_hi;
      const size_t t = vis ? (size_t)(slot0 + kb - w_lo) * H + h : 0;
      const i32x4 rs = buf_rsrc(a.dS + t * 1024, vis ? 2048u : 0u);
      const uint32_t dst = st + G::OFF_DS + (uint32_t)wave * 2048u;
      dma16_nt(rs, doff[0], dst);
      dma16_nt(rs, doff[1], dst + 1024);
    };

    f32x16 acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[o] = zero16();

    auto compute = [&](int kb, int buf) {
      if (kb < w_lo || kb > w_hi) return;
      const char* st = smem + buf * STAGE;
      const char* dt = st + G::OFF_DS + wave * 2048;
      // A operands: column l%32 (query ds_query(l%32)) of keys crow(j, hf),
      // then the same plus 16; the B operands take the same keys of K
      // every operand read before the products (in groups of GO output
      // tiles), so that one wait covers the reads' latency
      const h8 a0 = tr_operand<DT>(dt, 4 * hf, 8 + 4 * hf, 0, lane);
      const h8 a1 = tr_operand<DT>(dt, 16 + 4 * hf, 24 + 4 * hf, 0, lane);
#pragma unroll
      for (int o0 = 0; o0 < NO; o0 += G::GO) {
        h8 kv[G::GO][2];
#pragma unroll
        for (int o = o0; o < o0 + G::GO && o < NO; ++o) {
          kv[o - o0][0] = tr_operand<KT>(st, 4 * hf, 8 + 4 * hf, 32 * o, lane);
          kv[o - o0][1] = tr_operand<KT>(st, 16 + 4 * hf, 24 + 4 * hf, 32 * o, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int o = o0; o < o0 + G::GO && o < NO; ++o) acc[o] = mfma16(a0, kv[o - o0][0], acc[o]);
#pragma unroll
        for (int o = o0; o < o0 + G::GO && o < NO; ++o) acc[o] = mfma16(a1, kv[o - o0][1], acc[o]);
      }
    };

    // the ring: blocks i .. i + NBUF - 2 issued ahead of the compute of block i
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < n) issue(kb_first + k, k);
    for (int i = 0; i < n; ++i) {
      // this wave's loads of block i have landed once at most those of the
      // later issued blocks are outstanding
      wait_blocks<NBUF - 2, G::LPS>(min(NBUF - 2, n - 1 - i));
      // every wave: block i resident and done with block i - 1 (whose buffer
      // the next issue refills)
      asm volatile("s_barrier" ::: "memory");
      if (i + NBUF - 1 < n) issue(kb_first + i + NBUF - 1, (i + NBUF - 1) % NBUF);
      compute(kb_first + i, i % NBUF);
    }
    if constexpr (DP > 128 || (ROPE && NO % 2 == 0)) {
      // through LDS (free once every wave is done with the ring): the sums,
      // half the columns (an even number of output tiles: NO / 2 of them) at
      // a time, each wave into its own 32-row region;
      // then each lane adds whole 16-byte row chunks into dQ, a few chunks'
      // loads before their stores (above 128 columns the buffer form's
      // offsets do not fit beside the accumulators).  With RoPE each chunk
      // holds two whole column pairs, which it turns back before the store.
      constexpr int HALF = DP / 2;        // columns per half
      constexpr int LW = HALF + 4;        // floats per staged row: the half and 4 of padding
      constexpr int NCL = HALF / 4;       // 16-byte chunks per staged row
      constexpr int NPL = 32 * NCL / 64;  // chunks per lane
      constexpr int BT = NPL % 4 == 0 ? 4 : 2;  // chunks per batch
      static_assert(4 * 32 * LW * 4 <= NBUF * STAGE, "the staging regions fit the ring");
      static_assert(NPL % BT == 0, "whole batches");
      static_assert(NO % 2 == 0, "each half is NO / 2 whole output tiles");
      __syncthreads();
      float* const stg = reinterpret_cast<float*>(smem) + wave * 32 * LW;
      const size_t qstride = (size_t)H * a.d;
      const int r0 = i0 + 32 * wave, nrows = max(0, min(32, S - r0));
      const auto rq = out_rsrc(a.dQ + (size_t)h * a.d + (size_t)r0 * qstride,
                               nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * qstride + a.d) * 4) : 0u);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int oo = 0; oo < NO / 2; ++oo)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stg[ds_query(crow(r, hf)) * LW + 32 * oo + l32] = a.scale * acc[half * (NO / 2) + oo][r];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i0c = 0; i0c < NPL; i0c += BT) {
          uint32_t off[BT];
          f32x4 v[BT];
#pragma unroll
          for (int i = 0; i < BT; ++i) {
            const int c = lane + 64 * (i0c + i), row = c / NCL, col = HALF * half + 4 * (c % NCL);
            off[i] = (row < nrows && col < a.d) ? (uint32_t)(((size_t)row * qstride + col) * 4) : ATTN_BUF_OOB;
            v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off[i], 0, 0));
          }
#pragma unroll
          for (int i = 0; i < BT; ++i) {
            const int c = lane + 64 * (i0c + i), row = c / NCL, col = HALF * half + 4 * (c % NCL);
            v[i] += *reinterpret_cast<const f32x4*>(stg + row * LW + 4 * (c % NCL));
            if constexpr (ROPE) {
              const long long pos = (long long)r0 + row + a.rope_pos;
              const f32x2 p0 = rope_back_pair(v[i][0], v[i][1], pos, rope_freq(col, a.d, a.rope_base));
              const f32x2 p1 = rope_back_pair(v[i][2], v[i][3], pos, rope_freq(col + 2, a.d, a.rope_base));
              v[i] = f32x4{p0[0], p0[1], p1[0], p1[1]};
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[i]), rq, off[i], 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      dq_writeback<NO, ROPE, true>(a, acc, h, i0 + 32 * wave, hf, l32,
                                   [&](int r) { return ds_query(crow(r, hf)); });
    }
  };
  // longest rows first; paired: then the mirror tile
  const int first = qt_hi - (int)(blockIdx.x / H);
  const int second = mirror_tile(first, qt_hi + 1, a.pair);
  tile(first);
  if (second >= 0) {
    __syncthreads();  // every wave done with the ring and sMin of the first tile
    tile(second);
  }
}

// ---------------------------------------------------------------------------
// k_kv16: key-major, one workgroup per (128-key tile, KV head, head split,
// column part).  Wave w owns key block w (keys j0 + 32w + l%32) and holds its
// K and V rows in registers as the B operands of S = Q K^T and dP = dO V^T.
// Per visible 32-row query block and head of the split's share of the group,
// the Q and dO row tiles and the rows' LSE, D and seg stream through an LDS
// ring of NBUF stages (NBUF - 1 steps in flight), shared by the four waves.
// Each wave forms P and dS/scale = P (dP - D) in registers and accumulates
// dV += P^T dO and dK/scale += (dS/scale)^T Q over its part's output columns
// (the scale goes onto dK at the end), with the B operands read from the same
// row tiles by transposing loads.  A step whose every pair is visible skips
// the per-element mask: the block's largest document start (from k_prep) is
// staged with its rows.  Above 128 columns the output
// columns come in two parts, one workgroup each (both form S and dP), so that
// a wave's accumulators fit the register file.  The visible query blocks of
// the tile (blk_min <= last key, at or after the diagonal) come from 64-block
// ballots, the same in every wave.
// With one split the workgroup adds its sums into dK, dV; with several, each
// split writes its partial sums to its own slice of `part`, and k_sumparts
// adds the slices in split order (deterministic).
// ---------------------------------------------------------------------------
template <int DP>
struct KvGeom {
  static constexpr int NC = DP > 128 ? 2 : 1;  // output column parts
  static constexpr int DW = DP / NC;           // output columns per part
  static constexpr int NOW = DW / 32;          // 32-column output tiles per part
  using RT = Tile16<32, DP / 8>;
  static constexpr int OFF_DO = RT::BYTES;
  static constexpr int OFF_ROW = 2 * RT::BYTES;  // LSE*log2e, D, seg, block metadata (256 B each)
  static constexpr int STAGE = OFF_ROW + 4 * 256;
  static constexpr int NBUF = 4 * STAGE <= 150 * 1024 ? 4 : 3 * STAGE <= 150 * 1024 ? 3 : 2;
  static constexpr int LPS = 2 * RT::CPW + 1;  // loads per wave per step
  static_assert(DW % 32 == 0, "whole output tiles per part");
  static_assert((NBUF - 2) * LPS < 64, "loads in flight fit vmcnt");
};

template <int DP, bool ROPE>
__global__ __launch_bounds__(256, 1) void k_kv16(F16Args a) {
  using G = KvGeom<DP>;
  using RT = typename G::RT;
  constexpr int NT = DP / 16, NOW = G::NOW, NBUF = G::NBUF, STAGE = G::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H, KV = a.KV;
  const int g = H / KV, gs = g / a.splits;  // heads of the group per split
  // grid position -> (KV head, column part, split, first key tile).  With two
  // column parts, those of one (tile, KV head, split) run 8 blocks apart:
  // blocks are dispatched round-robin over the 8 XCDs, so both land on the
  // same XCD at about the same time, and the second finds the Q and dO
  // tiles the first brought into that XCD's L2.  (The grid is then padded
  // to a multiple of 16 blocks; the padding exits here.)
  int b = (int)blockIdx.x, cpart = 0;
  if constexpr (G::NC == 2) {
    cpart = (b >> 3) & 1;
    b = ((b >> 4) << 3) | (b & 7);
    if (b >= a.kv_work) return;
  }
  const int kvh = b % KV;
  b /= KV;
  const int split = b % a.splits;
  const int first_tile = b / a.splits;
  const int nblk = (S + 31) / 32;
  const float sc2 = a.scale * ATTN_LOG2E;
  const uint32_t smem0 = lds_addr(smem);
  Loader16<32, DP / 8> ldr;
  ldr.init(DP * 2, wave, lane);

  auto tile = [&](const int kt) __attribute__((always_inline)) {
    const int j0 = kt * 128;
    const int key = j0 + 32 * wave + l32;  // < Sp: the copies hold zero rows up to Sp
    h8 kreg[NT], vreg[NT];
    const size_t boff = ((size_t)kvh * a.Sp + key) * DP + 8 * hf;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kreg[t] = *reinterpret_cast<const h8*>(a.Kh + boff + 16 * t);
      vreg[t] = *reinterpret_cast<const h8*>(a.Vh + boff + 16 * t);
    }
    // land them now, where the compiler sees it: otherwise it waits for them
    // inside the step loop, on a counter that also counts the ring's loads
    wait_vm<0>();
    // the accumulators live in AGPRs for the whole tile (the matrix cores read
    // and write them there; pinned so that no step copies them to VGPRs)
    f32x16 accK[NOW], accV[NOW];
#pragma unroll
    for (int o = 0; o < NOW; ++o) {
      accK[o] = zero16();
      accV[o] = zero16();
      asm volatile("" : "+a"(accK[o]), "+a"(accV[o]));
    }

    // visible query blocks: qb >= j0/32 whose smallest document start is at or
    // before the tile's last key
    const uint32_t khi = (uint32_t)min(j0 + 127, S - 1);
    int segb = j0 >> 5;
    auto seg_mask = [&](int bb) -> uint64_t {
      const int qb = bb + lane;
      return __ballot(qb < nblk && a.blk_min[qb] <= khi);
    };
    uint64_t mask = segb < nblk ? seg_mask(segb) : 0ull;
    // smallest visible block after `prev` (-1 when none is left)
    auto next_block = [&](int prev) -> int {
      if (prev >= segb) {
        const int sh = prev - segb + 1;
        mask = sh >= 64 ? 0ull : (mask >> sh) << sh;
      }
      while (mask == 0ull) {
        segb += 64;
        if (segb >= nblk) return -1;
        mask = seg_mask(segb);
      }
      return segb + (int)__builtin_ctzll(mask);
    };
    // the step after (qb, hh): the next head of the split, then the next block
    auto next_step = [&](int& qb, int& hh) {
      if (qb < 0) return;
      if (++hh == gs) {
        hh = 0;
        qb = next_block(qb);
      }
    };

    auto issue = [&](int qb, int hh, int buf) {
      const int head = kvh * g + split * gs + hh;
      const uint32_t st = smem0 + (uint32_t)(buf * STAGE);
      const size_t roff = ((size_t)head * a.Sp + (size_t)qb * 32) * DP;
      ldr.load(buf_rsrc(a.Qh + roff, 32 * DP * 2), st, wave);
      ldr.load(buf_rsrc(a.dOh + roff, 32 * DP * 2), st + G::OFF_DO, wave);
      // LSE, D and seg of the block's rows (lanes 0..31; the rest deposit
      // zeros), and the block's metadata (wave 3: meta_off)
      const int rows = min(32, S - qb * 32);
      const bool rok = hf == 0 && l32 < rows;
      const uint32_t roff4 = rok ? (uint32_t)(l32 * H + head) * 4u : ATTN_BUF_OOB;
      const uint32_t rbytes = (uint32_t)(rows * H * 4);
      if (wave == 0) dma4(buf_rsrc(a.LSE2 + (size_t)qb * 32 * H, rbytes), roff4, st + G::OFF_ROW);
      else if (wave == 1) dma4(buf_rsrc(a.D + (size_t)qb * 32 * H, rbytes), roff4, st + G::OFF_ROW + 256);
      else if (wave == 2)
        dma4(buf_rsrc(a.seg ? (const void*)(a.seg + (size_t)qb * 32) : (const void*)a.LSE,
                      a.seg ? (uint32_t)rows * 4u : 0u),
             rok ? (uint32_t)l32 * 4u : ATTN_BUF_OOB, st + G::OFF_ROW + 512);
      else dma4(buf_rsrc(a.blk_min, a.meta_bytes), meta_off(a, qb, lane), st + G::OFF_ROW + 768);
    };

    auto compute = [&](int qb, int hh, int buf) {
      const int q0 = qb * 32, k0 = j0 + 32 * wave;
      if (k0 > q0 + 31) return;  // every key of the block after every query
      const char* st = smem + buf * STAGE;
      // every pair visible: keys at or before every query, every row inside
      // S, and no document start of the rows after the first key (the
      // block's largest seg is staged with its rows)
      const uint32_t mx = __builtin_amdgcn_readfirstlane(
          *reinterpret_cast<const uint32_t*>(st + G::OFF_ROW + 768));
      const bool full = (k0 + 31 <= q0) & (q0 + 31 < S) & (mx <= (uint32_t)k0);
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s = mfma16(*reinterpret_cast<const h8*>(st + RT::at(l32, 2 * t + hf)), kreg[t], s);
        dp = mfma16(*reinterpret_cast<const h8*>(st + G::OFF_DO + RT::at(l32, 2 * t + hf)), vreg[t],
                    dp);
      }
      // LSE * log2(e) and D of this lane's rows crow(r, hf): rows 8(r/4) +
      // 4hf + r%4, four 16-byte reads each
      float lse[16], dv[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int row0 = 8 * a4 + 4 * hf;
        const float4 l4 = *reinterpret_cast<const float4*>(st + G::OFF_ROW + 4 * row0);
        const float4 d4 = *reinterpret_cast<const float4*>(st + G::OFF_ROW + 256 + 4 * row0);
        lse[4 * a4] = l4.x; lse[4 * a4 + 1] = l4.y; lse[4 * a4 + 2] = l4.z; lse[4 * a4 + 3] = l4.w;
        dv[4 * a4] = d4.x; dv[4 * a4 + 1] = d4.y; dv[4 * a4 + 2] = d4.z; dv[4 * a4 + 3] = d4.w;
      }
      // P, and dS/scale = P (dP - D) (the scale goes onto dK at the end)
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse[r]));
          s[r] = p;
          dp[r] = p * (dp[r] - dv[r]);
        }
      } else {
        uint32_t sg[16];  // seg of the rows
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const uint4 s4 =
              *reinterpret_cast<const uint4*>(st + G::OFF_ROW + 512 + 4 * (8 * a4 + 4 * hf));
          sg[4 * a4] = s4.x; sg[4 * a4 + 1] = s4.y; sg[4 * a4 + 2] = s4.z; sg[4 * a4 + 3] = s4.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = q0 + crow(r, hf);
          const bool vis = (qq < S) & (key <= qq) & ((uint32_t)key >= sg[r]);
          const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse[r]));
          const float p = vis ? e : 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - dv[r]);
        }
      }
      const h8 p0 = pack8(s, 0), p1 = pack8(s, 1), d0 = pack8(dp, 0), d1 = pack8(dp, 1);
      if (a.dS && cpart == 0) {
        _Float16* t = ds_tile(a, *reinterpret_cast<const uint4*>(st + G::OFF_ROW + 768), k0 >> 5,
                              kvh * g + split * gs + hh);
        if (t) ds_write(t, lane, d0, d1);
      }
      // B operands from the Q and dO row tiles (transposing loads): the k
      // order of p0 / d0 is queries crow(j, hf), j = 0..7, i.e. rows 4 hf ..
      // 4 hf + 3 then 8 + 4 hf .. ; of p1 / d1 the same plus 16
#pragma unroll
      for (int o = 0; o < NOW; ++o) {
        const int n0 = cpart * G::DW + 32 * o;
        const h8 ov0 = tr_operand<RT>(st + G::OFF_DO, 4 * hf, 8 + 4 * hf, n0, lane);
        const h8 ov1 = tr_operand<RT>(st + G::OFF_DO, 16 + 4 * hf, 24 + 4 * hf, n0, lane);
        const h8 qv0 = tr_operand<RT>(st, 4 * hf, 8 + 4 * hf, n0, lane);
        const h8 qv1 = tr_operand<RT>(st, 16 + 4 * hf, 24 + 4 * hf, n0, lane);
        accV[o] = mfma16(p0, ov0, accV[o]);
        accV[o] = mfma16(p1, ov1, accV[o]);
        accK[o] = mfma16(d0, qv0, accK[o]);
        accK[o] = mfma16(d1, qv1, accK[o]);
        asm volatile("" : "+a"(accK[o]), "+a"(accV[o]));
      }
    };

    // the ring: steps i .. i + NBUF - 2 issued ahead of the compute of step i
    int rq[NBUF], rh[NBUF];  // issued steps, oldest first (rq = -1: none)
    rq[0] = next_block(-1);
    rh[0] = 0;
#pragma unroll
    for (int k = 1; k < NBUF; ++k) {
      rq[k] = rq[k - 1];
      rh[k] = rh[k - 1];
      next_step(rq[k], rh[k]);
    }
    // rq[NBUF - 1] is the first step not yet issued
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (rq[k] >= 0) issue(rq[k], rh[k], k);
    int buf = 0;
    while (rq[0] >= 0) {
      // this wave's loads of step i have landed once at most those of the
      // later issued steps are outstanding
      int ahead = 0;
#pragma unroll
      for (int k = 1; k < NBUF - 1; ++k) ahead += rq[k] >= 0;
      if constexpr (NBUF >= 4) {
        if (ahead >= 2) wait_vm<2 * G::LPS>();
        else if (ahead == 1) wait_vm<G::LPS>();
        else wait_vm<0>();
      } else if constexpr (NBUF == 3) {
        if (ahead >= 1) wait_vm<G::LPS>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
      // every wave: step i resident and done with step i - 1 (whose buffer the
      // next issue refills)
      asm volatile("s_barrier" ::: "memory");
      if (rq[NBUF - 1] >= 0) issue(rq[NBUF - 1], rh[NBUF - 1], (buf + NBUF - 1) % NBUF);
      compute(rq[0], rh[0], buf);
      // shift the ring
      int nq = rq[NBUF - 1], nh = rh[NBUF - 1];
      next_step(nq, nh);
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k) {
        rq[k] = rq[k + 1];
        rh[k] = rh[k + 1];
      }
      rq[NBUF - 1] = nq;
      rh[NBUF - 1] = nh;
      buf = (buf + 1) % NBUF;
    }
    __syncthreads();  // every wave done with the ring before it is reused

    // rows key j0 + 32w + crow(r, hf), the part's columns: += into dK, dV (one
    // split; with RoPE dK = R^T (dK + scale * accK), the pair partner in lane
    // l ^ 1), or this split's partial sums into part (several; k_sumparts
    // then adds and rotates).  Through buffers over the wave's rows: rows
    // past S and columns past head_dim read zero and drop their stores.
    const size_t kstride = (size_t)KV * a.d;
    const size_t slice = (size_t)S * kstride;
    const int r0 = j0 + 32 * wave, nrows = max(0, min(32, S - r0));
    const uint32_t rbytes =
        nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * kstride + a.d) * 4) : 0u;
    const size_t base = (size_t)kvh * a.d + (size_t)r0 * kstride;
    const auto rK = wave_rsrc((a.splits == 1 ? a.dK : a.part + (size_t)(2 * split) * slice) + base,
                              rbytes);
    const auto rV = wave_rsrc((a.splits == 1 ? a.dV : a.part + (size_t)(2 * split + 1) * slice) + base,
                              rbytes);
    const bool add = a.splits == 1;
    // eight rows at a time: their loads, then their adds and stores
#pragma unroll
    for (int o = 0; o < NOW; ++o) {
      const int col = cpart * G::DW + 32 * o + l32;
      const double fq = ROPE ? rope_freq(col, a.d, a.rope_base) : 0.0;
#pragma unroll
      for (int q0 = 0; q0 < 16; q0 += 8) {
        uint32_t off[8];
        float vk[8], vv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int rr = crow(q0 + r, hf);
          off[r] = (rr < nrows && col < a.d) ? (uint32_t)(((size_t)rr * kstride + col) * 4) : ATTN_BUF_OOB;
          vk[r] = add ? buf_ld(rK, off[r]) : 0.f;
          vv[r] = add ? buf_ld(rV, off[r]) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          vk[r] += a.scale * accK[o][q0 + r];
          vv[r] += accV[o][q0 + r];
          if constexpr (ROPE) {
            if (add)
              vk[r] = rope_back(vk[r], __shfl_xor(vk[r], 1), col,
                                (long long)r0 + crow(q0 + r, hf) + a.rope_pos, fq);
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          buf_st(rK, off[r], vk[r]);
          buf_st(rV, off[r], vv[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // low key tiles (most queries) first; paired: then the mirror tile
  const int first = first_tile;
  const int second = mirror_tile(first, (S + 127) / 128, a.pair);
  tile(first);
  if (second >= 0) tile(second);
}

// ---------------------------------------------------------------------------
// k_kv16r: the key-major pass of k_kv16 with the work of each key block
// split by role over two waves, so that two waves share each SIMD and one
// wave's products run while the other exponentiates.  One workgroup of eight
// waves per (128-key tile, KV head, head split, column part), as k_kv16.
// Waves 0..3 (role P) own key block w: per step they form S = Q K^T, P
// (masked), write P in fp16 to LDS and accumulate dV += P^T dO.  Waves 4..7
// (role dS) own key block w - 4 and run one step behind: they form
// dP = dO V^T, read that step's P back, form dS/scale = P (dP - D) and
// accumulate dK/scale += (dS/scale)^T Q.  P reaches dS rounded to fp16, as
// it enters dV.  A step's stage stays in the ring until the lagging role has
// used it; one barrier per step orders the stage loads, the P hand-over and
// the reuse of both.  The role-dS waves issue the ring's loads.
// ---------------------------------------------------------------------------
template <int DP>
struct KvrGeom {
  static constexpr int NC = DP > 128 ? 2 : 1;  // output column parts
  static constexpr int DW = DP / NC;
  static constexpr int NOW = DW / 32;
  using RT = Tile16<32, DP / 8>;
  static constexpr int OFF_DO = RT::BYTES;
  static constexpr int OFF_ROW = 2 * RT::BYTES;  // LSE*log2e, D, seg, block metadata (256 B each)
  static constexpr int STAGE = OFF_ROW + 4 * 256;
  static constexpr int PBYTES = 2 * 4 * 2048;    // P hand-over: [step parity][key block]
  static constexpr int NBUF = (150 * 1024 - PBYTES) / STAGE >= 6 ? 6 : (150 * 1024 - PBYTES) / STAGE;
  static constexpr int LPS = 2 * RT::CPW + 1;    // loads per loading wave per step
  static_assert(NBUF >= 3, "the ring holds the lagging step, the current one and one ahead");
  static_assert((NBUF - 3) * LPS < 64, "loads in flight fit vmcnt");
};

template <int DP, bool ROPE>
__global__ __launch_bounds__(512, 1) void k_kv16r(F16Args a) {
  using G = KvrGeom<DP>;
  using RT = typename G::RT;
  constexpr int NT = DP / 16, NOW = G::NOW, NBUF = G::NBUF, STAGE = G::STAGE;
  // output tiles whose B operands are read before the exponentials (the rest
  // right after them): all of them up to 64 columns; at 96 and 128 columns
  // prefetching spills registers, and none is read ahead (measured at 128
  // columns: no prefetch 0.410 ms, one tile 0.415, two 0.432)
  constexpr int PF = NOW <= 2 ? NOW : 0;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE + G::PBYTES];
  char* const pbuf0 = smem + NBUF * STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2, kb = wave & 3;  // role 0: S, P, dV; role 1: dP, dS, dK
  const int hf = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H, KV = a.KV;
  const int g = H / KV, gs = g / a.splits;
  int b = (int)blockIdx.x, cpart = 0;
  if constexpr (G::NC == 2) {
    cpart = (b >> 3) & 1;
    b = ((b >> 4) << 3) | (b & 7);
    if (b >= a.kv_work) return;
  }
  const int kvh = b % KV;
  b /= KV;
  const int split = b % a.splits;
  const int first_tile = b / a.splits;
  const int nblk = (S + 31) / 32;
  const float sc2 = a.scale * ATTN_LOG2E;
  const uint32_t smem0 = lds_addr(smem);
  Loader16<32, DP / 8> ldr;
  ldr.init(DP * 2, kb, lane);  // used by the role-dS waves (loader index kb)

  auto tile = [&](const int kt) __attribute__((always_inline)) {
    const int j0 = kt * 128;
    const int k0 = j0 + 32 * kb;
    const int key = k0 + l32;  // < Sp: the copies hold zero rows up to Sp
    // role P holds its keys' K rows (B operand of S = Q K^T), role dS their V
    // rows (B operand of dP = dO V^T)
    // (loaded once the ring's first steps are found, so that they are not
    // live across that search)
    h8 xreg[NT];
    f32x16 acc[NOW];  // role P: dV; role dS: dK / scale
#pragma unroll
    for (int o = 0; o < NOW; ++o) {
      acc[o] = zero16();
      asm volatile("" : "+v"(acc[o]));
    }

    const uint32_t khi = (uint32_t)min(j0 + 127, S - 1);
    int segb = j0 >> 5;
    auto seg_mask = [&](int bb) -> uint64_t {
      const int qb = bb + lane;
      return __ballot(qb < nblk && a.blk_min[qb] <= khi);
    };
    uint64_t mask = segb < nblk ? seg_mask(segb) : 0ull;
    auto next_block = [&](int prev) -> int {
      if (prev >= segb) {
        const int sh = prev - segb + 1;
        mask = sh >= 64 ? 0ull : (mask >> sh) << sh;
      }
      while (mask == 0ull) {
        segb += 64;
        if (segb >= nblk) return -1;
        mask = seg_mask(segb);
      }
      return segb + (int)__builtin_ctzll(mask);
    };
    auto next_step = [&](int& qb, int& hh) {
      if (qb < 0) return;
      if (++hh == gs) {
        hh = 0;
        qb = next_block(qb);
      }
    };

    // the role-dS waves load a step's stage (loader wave index kb)
    auto issue = [&](int qb, int hh, int buf) {
      const int head = kvh * g + split * gs + hh;
      const uint32_t st = smem0 + (uint32_t)(buf * STAGE);
      const size_t roff = ((size_t)head * a.Sp + (size_t)qb * 32) * DP;
      ldr.load(buf_rsrc(a.Qh + roff, 32 * DP * 2), st, kb);
      ldr.load(buf_rsrc(a.dOh + roff, 32 * DP * 2), st + G::OFF_DO, kb);
      const int rows = min(32, S - qb * 32);
      const bool rok = hf == 0 && l32 < rows;
      const uint32_t roff4 = rok ? (uint32_t)(l32 * H + head) * 4u : ATTN_BUF_OOB;
      const uint32_t rbytes = (uint32_t)(rows * H * 4);
      if (kb == 0) dma4(buf_rsrc(a.LSE2 + (size_t)qb * 32 * H, rbytes), roff4, st + G::OFF_ROW);
      else if (kb == 1) dma4(buf_rsrc(a.D + (size_t)qb * 32 * H, rbytes), roff4, st + G::OFF_ROW + 256);
      else if (kb == 2)
        dma4(buf_rsrc(a.seg ? (const void*)(a.seg + (size_t)qb * 32) : (const void*)a.LSE,
                      a.seg ? (uint32_t)rows * 4u : 0u),
             rok ? (uint32_t)l32 * 4u : ATTN_BUF_OOB, st + G::OFF_ROW + 512);
      else dma4(buf_rsrc(a.blk_min, a.meta_bytes), meta_off(a, qb, lane), st + G::OFF_ROW + 768);
    };

    // role P, step (qb, buf): S, P (written to the hand-over slot), dV.  The
    // operand reads are issued ahead of their products (scheduling barriers
    // keep the compiler from sinking them): all of S's, then, before the
    // exponentials, all of dV's
    auto compute_p = [&](int qb, int buf, int par) {
      const int q0 = qb * 32;
      if (k0 > q0 + 31) return;  // every key of the block after every query
      const char* st = smem + buf * STAGE;
      const uint32_t mx = __builtin_amdgcn_readfirstlane(
          *reinterpret_cast<const uint32_t*>(st + G::OFF_ROW + 768));
      const bool full = (k0 + 31 <= q0) & (q0 + 31 < S) & (mx <= (uint32_t)k0);
      // S's operand reads in groups of at most 8, each issued ahead of its products
      f32x16 s = zero16();
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += 8) {
        h8 qop[8];
#pragma unroll
        for (int t = 0; t < 8 && t0 + t < NT; ++t)
          qop[t] = *reinterpret_cast<const h8*>(st + RT::at(l32, 2 * (t0 + t) + hf));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 8 && t0 + t < NT; ++t) s = mfma16(qop[t], xreg[t0 + t], s);
      }
      h8 ov[NOW][2];
      auto read_ov = [&](int o) __attribute__((always_inline)) {
        const int n0 = cpart * G::DW + 32 * o;
        ov[o][0] = tr_operand<RT>(st + G::OFF_DO, 4 * hf, 8 + 4 * hf, n0, lane);
        ov[o][1] = tr_operand<RT>(st + G::OFF_DO, 16 + 4 * hf, 24 + 4 * hf, n0, lane);
      };
#pragma unroll
      for (int o = 0; o < PF; ++o) read_ov(o);
      float lse[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 l4 = *reinterpret_cast<const float4*>(st + G::OFF_ROW + 4 * (8 * a4 + 4 * hf));
        lse[4 * a4] = l4.x; lse[4 * a4 + 1] = l4.y; lse[4 * a4 + 2] = l4.z; lse[4 * a4 + 3] = l4.w;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse[r]));
      } else {
        uint32_t sg[16];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const uint4 s4 =
              *reinterpret_cast<const uint4*>(st + G::OFF_ROW + 512 + 4 * (8 * a4 + 4 * hf));
          sg[4 * a4] = s4.x; sg[4 * a4 + 1] = s4.y; sg[4 * a4 + 2] = s4.z; sg[4 * a4 + 3] = s4.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = q0 + crow(r, hf);
          const bool vis = (qq < S) & (key <= qq) & ((uint32_t)key >= sg[r]);
          const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse[r]));
          s[r] = vis ? e : 0.f;
        }
      }
      const h8 p0 = pack8(s, 0), p1 = pack8(s, 1);
      char* pb = pbuf0 + (par * 4 + kb) * 2048;
      *reinterpret_cast<h8*>(pb + 16 * lane) = p0;
      *reinterpret_cast<h8*>(pb + 1024 + 16 * lane) = p1;
#pragma unroll
      for (int o = PF; o < NOW; ++o) read_ov(o);
#pragma unroll
      for (int o = 0; o < NOW; ++o) {
        acc[o] = mfma16(p0, ov[o][0], acc[o]);
        acc[o] = mfma16(p1, ov[o][1], acc[o]);
        asm volatile("" : "+v"(acc[o]));
      }
    };

    // role dS, in the order that puts its products beside role P's
    // exponentials: first dS/scale = P (dP - D) of step i - 1 and its
    // products dK/scale += (dS/scale)^T Q (ds_finish), then dP = dO V^T of
    // step i (ds_start), kept in registers for the next iteration
    f32x16 dpc = zero16();
    auto ds_start = [&](int qb, int buf) {
      if (k0 > qb * 32 + 31) return;
      const char* st = smem + buf * STAGE;
      dpc = zero16();
      // (groups of 4: with 8 the role's registers spill at 128 columns)
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += 4) {
        h8 dop[4];
#pragma unroll
        for (int t = 0; t < 4 && t0 + t < NT; ++t)
          dop[t] = *reinterpret_cast<const h8*>(st + G::OFF_DO + RT::at(l32, 2 * (t0 + t) + hf));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4 && t0 + t < NT; ++t) dpc = mfma16(dop[t], xreg[t0 + t], dpc);
      }
    };
    auto ds_finish = [&](int qb, int hh, int buf, int par) {
      if (k0 > qb * 32 + 31) return;
      const char* st = smem + buf * STAGE;
      h8 qv[NOW][2];
      auto read_qv = [&](int o) __attribute__((always_inline)) {
        const int n0 = cpart * G::DW + 32 * o;
        qv[o][0] = tr_operand<RT>(st, 4 * hf, 8 + 4 * hf, n0, lane);
        qv[o][1] = tr_operand<RT>(st, 16 + 4 * hf, 24 + 4 * hf, n0, lane);
      };
      const char* pb = pbuf0 + (par * 4 + kb) * 2048;
      const h8 p0 = *reinterpret_cast<const h8*>(pb + 16 * lane);
      const h8 p1 = *reinterpret_cast<const h8*>(pb + 1024 + 16 * lane);
      // the block's metadata for the dS store, read with the step's other LDS reads
      const uint4 meta = *reinterpret_cast<const uint4*>(st + G::OFF_ROW + 768);
      float dv[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 d4 =
            *reinterpret_cast<const float4*>(st + G::OFF_ROW + 256 + 4 * (8 * a4 + 4 * hf));
        dv[4 * a4] = d4.x; dv[4 * a4 + 1] = d4.y; dv[4 * a4 + 2] = d4.z; dv[4 * a4 + 3] = d4.w;
      }
#pragma unroll
      for (int o = 0; o < PF; ++o) read_qv(o);
      __builtin_amdgcn_sched_barrier(0);
      const f32x8 pf0 = __builtin_convertvector(p0, f32x8);
      const f32x8 pf1 = __builtin_convertvector(p1, f32x8);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = (r < 8 ? pf0[r] : pf1[r - 8]) * (dpc[r] - dv[r]);
      const h8 d0 = pack8(ds, 0), d1 = pack8(ds, 1);
#pragma unroll
      for (int o = PF; o < NOW; ++o) read_qv(o);
#pragma unroll
      for (int o = 0; o < NOW; ++o) {
        acc[o] = mfma16(d0, qv[o][0], acc[o]);
        acc[o] = mfma16(d1, qv[o][1], acc[o]);
        asm volatile("" : "+v"(acc[o]));
      }
      // the tile for the query-major dQ pass (after the products: stored
      // before them, or through role P, the role's registers spilled or the
      // hand-over's LDS traffic cost more).  These stores join the wave's
      // count of memory operations, so the ring's waits for its stage loads,
      // which count only loads, wait for somewhat more than they need.
      if (a.dS) {
        _Float16* t = ds_tile(a, meta, k0 >> 5, kvh * g + split * gs + hh);
        if (t) ds_write(t, lane, d0, d1);
      }
    };

    // the ring: role P computes step i in stage buf, role dS step i - 1 in
    // stage pbuf; steps i + 1 .. i + NBUF - 3 are in flight, and after the
    // barrier step i + NBUF - 2 is issued into the stage of step i - 2.  Each
    // role runs its own copy of the loop (same steps, same barriers), so that
    // each loop has a single path through its products.
    auto ring = [&](auto&& work) __attribute__((always_inline)) {
      int rq[NBUF - 1], rh[NBUF - 1];  // steps i .. i + NBUF - 2 (rq = -1: none)
      rq[0] = next_block(-1);
      rh[0] = 0;
#pragma unroll
      for (int k = 1; k < NBUF - 1; ++k) {
        rq[k] = rq[k - 1];
        rh[k] = rh[k - 1];
        next_step(rq[k], rh[k]);
      }
      const size_t boff = ((size_t)kvh * a.Sp + key) * DP + 8 * hf;
      const _Float16* xsrc = role == 0 ? a.Kh : a.Vh;
#pragma unroll
      for (int t = 0; t < NT; ++t) xreg[t] = *reinterpret_cast<const h8*>(xsrc + boff + 16 * t);
      wait_vm<0>();
      if (role == 1) {
#pragma unroll
        for (int k = 0; k < NBUF - 2; ++k)
          if (rq[k] >= 0) issue(rq[k], rh[k], k);
      }
      int pq = -1, ph = 0, pbuf = 0, buf = 0, par = 0;
      while (rq[0] >= 0 || pq >= 0) {
        if (role == 1) {
          // this wave's loads of step i have landed once at most those of the
          // later issued steps (i + 1 .. i + NBUF - 3) are outstanding (the
          // dS stores issued since count too, so these waits cover a little
          // more than step i: counting the stores exactly gained nothing)
          int ahead = 0;
#pragma unroll
          for (int k = 1; k < NBUF - 2; ++k) ahead += rq[k] >= 0;
          if constexpr (NBUF >= 6) {
            if (ahead >= 3) wait_vm<3 * G::LPS>();
            else if (ahead == 2) wait_vm<2 * G::LPS>();
            else if (ahead == 1) wait_vm<G::LPS>();
            else wait_vm<0>();
          } else if constexpr (NBUF == 5) {
            if (ahead >= 2) wait_vm<2 * G::LPS>();
            else if (ahead == 1) wait_vm<G::LPS>();
            else wait_vm<0>();
          } else if constexpr (NBUF == 4) {
            if (ahead >= 1) wait_vm<G::LPS>();
            else wait_vm<0>();
          } else {
            wait_vm<0>();
          }
        }
        // step i resident; P of step i - 1 written; step i - 2's stage and
        // hand-over slot done with
        asm volatile("s_barrier" ::: "memory");
        if (role == 1 && rq[NBUF - 2] >= 0)
          issue(rq[NBUF - 2], rh[NBUF - 2], (buf + NBUF - 2) % NBUF);
        work(rq[0], buf, par, pq, ph, pbuf);
        pq = rq[0];
        ph = rh[0];
        pbuf = buf;
        int nq = rq[NBUF - 2], nh = rh[NBUF - 2];
        next_step(nq, nh);
#pragma unroll
        for (int k = 0; k < NBUF - 2; ++k) {
          rq[k] = rq[k + 1];
          rh[k] = rh[k + 1];
        }
        rq[NBUF - 2] = nq;
        rh[NBUF - 2] = nh;
        buf = (buf + 1) % NBUF;
        par ^= 1;
      }
    };
    if (role == 0)
      ring([&](int q, int bf, int pr, int, int, int) {
        if (q >= 0) compute_p(q, bf, pr);
      });
    else
      ring([&](int q, int bf, int pr, int pq, int ph, int pbf) {
        if (pq >= 0) ds_finish(pq, ph, pbf, pr ^ 1);
        if (q >= 0) ds_start(q, bf);
      });
    __syncthreads();  // every wave done with the ring before it is reused

    // rows key k0 + crow(r, hf), the part's columns: role P adds dV, role dS
    // scale * dK (with RoPE dK = R^T (dK + scale * acc)), or this split's
    // partial sums into part
    const size_t kstride = (size_t)KV * a.d;
    const size_t slice = (size_t)S * kstride;
    const int nrows = max(0, min(32, S - k0));
    const uint32_t rbytes =
        nrows > 0 ? (uint32_t)(((size_t)(nrows - 1) * kstride + a.d) * 4) : 0u;
    const size_t base = (size_t)kvh * a.d + (size_t)k0 * kstride;
    float* const whole = role == 0 ? a.dV : a.dK;
    const auto rO = wave_rsrc((a.splits == 1 ? whole : a.part + (size_t)(2 * split + (role == 0)) * slice) +
                                  base,
                              rbytes);
    const float f = role == 0 ? 1.f : a.scale;
    const bool add = a.splits == 1;
    // eight rows at a time: their loads, then their adds and stores.  At
    // 128 columns the registers hold only one element at a time (the
    // batched form spilled inside the step loop): a load, add and store each
#pragma unroll
    for (int o = 0; o < NOW && DP < 128; ++o) {
      const int col = cpart * G::DW + 32 * o + l32;
      const double fq = ROPE ? rope_freq(col, a.d, a.rope_base) : 0.0;
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 8) {
        uint32_t off[8];
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int rr = crow(r0 + r, hf);
          off[r] = (rr < nrows && col < a.d) ? (uint32_t)(((size_t)rr * kstride + col) * 4) : ATTN_BUF_OOB;
          v[r] = add ? buf_ld(rO, off[r]) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          v[r] += f * acc[o][r0 + r];
          if constexpr (ROPE) {
            if (add) {
              const float partner = __shfl_xor(v[r], 1);
              if (role == 1)
                v[r] = rope_back(v[r], partner, col, (long long)k0 + crow(r0 + r, hf) + a.rope_pos, fq);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) buf_st(rO, off[r], v[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int o = 0; o < NOW && DP == 128; ++o) {
      const int col = cpart * G::DW + 32 * o + l32;
      const double fq = ROPE ? rope_freq(col, a.d, a.rope_base) : 0.0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = crow(r, hf);
        const uint32_t off = (rr < nrows && col < a.d) ? (uint32_t)(((size_t)rr * kstride + col) * 4)
                                                       : ATTN_BUF_OOB;
        if (add) {
          float v = buf_ld(rO, off) + f * acc[o][r];
          if constexpr (ROPE) {
            const float partner = __shfl_xor(v, 1);
            if (role == 1) v = rope_back(v, partner, col, (long long)k0 + rr + a.rope_pos, fq);
          }
          buf_st(rO, off, v);
        } else {
          buf_st(rO, off, f * acc[o][r]);
        }
      }
    }
  };
  const int first = first_tile;
  const int second = mirror_tile(first, (S + 127) / 128, a.pair);
  tile(first);
  if (second >= 0) tile(second);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int DP>
static attn_status_t launch_f16(const F16Args& f, const CvtArgs& c, const float* O, const float* dO,
                                hipStream_t st) {
  auto blocks = [&](int ntiles) { return f.pair ? (ntiles + 1) / 2 : ntiles; };
  const int nb = f.Sp / 32;
  const long long ncvt = 2ll * nb * f.H + 2ll * nb * f.KV;
  attn_status_t rc = profile_mark(st, true);
  if (rc != ATTN_OK) return rc;
  hipLaunchKernelGGL(k_cvt16<DP>, dim3((unsigned)ncvt), dim3(256), 0, st, c);
  rc = hip_check(hipGetLastError(), "launching k_cvt16");
  if (rc != ATTN_OK) return rc;
  const int nqt = blocks((f.S + 127) / 128);
  if (O) {
    rc = launch_rowdot(O, dO, f.D, (long long)f.S * f.H, f.d, st);
  } else {
    hipLaunchKernelGGL((k_q16<DP, true, false>), dim3(nqt * f.H), dim3(256), 0, st, f);
    rc = hip_check(hipGetLastError(), "launching k_q16 (row term)");
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc != ATTN_OK) return rc;
  const int kv_grid = KvGeom<DP>::NC == 2 ? (f.kv_work + 7) / 8 * 16 : f.kv_work;
  // the role-split key-major kernel where its 256 registers per wave hold
  // the work without spilling (up to 128 columns; at 128 with RoPE the
  // write-back's rotation spills, 0.535 against 0.452 ms); else one wave per
  // key block.  With split heads the pass writes unrotated partial sums and
  // k_sumparts rotates the total, so there the kernel without the rotation
  // serves RoPE calls too
  if constexpr (DP <= 96) {
    if (f.rope && f.splits == 1)
      hipLaunchKernelGGL((k_kv16r<DP, true>), dim3(kv_grid), dim3(512), 0, st, f);
    else
      hipLaunchKernelGGL((k_kv16r<DP, false>), dim3(kv_grid), dim3(512), 0, st, f);
  } else if (DP == 128 && (!f.rope || f.splits > 1)) {
    hipLaunchKernelGGL((k_kv16r<128, false>), dim3(kv_grid), dim3(512), 0, st, f);
  } else {
    if (f.rope)
      hipLaunchKernelGGL((k_kv16<DP, true>), dim3(kv_grid), dim3(256), 0, st, f);
    else
      hipLaunchKernelGGL((k_kv16<DP, false>), dim3(kv_grid), dim3(256), 0, st, f);
  }
  rc = hip_check(hipGetLastError(), "launching k_kv16");
  if (rc == ATTN_OK && f.splits > 1) {
    rc = launch_sumparts(f.part, f.splits, f.S, f.KV * f.d, (long long)f.KV * f.d, f.dK, f.dV, st,
                         f.rope, f.d, f.rope_pos, f.rope_base);
  }
  if (rc == ATTN_OK) rc = profile_mark(st);
  if (rc != ATTN_OK) return rc;
  // dQ from the stored dS tiles, or with dS formed again from the scores
  if (f.dS && f.rope)
    hipLaunchKernelGGL((k_dqs16<DP, true>), dim3(nqt * f.H), dim3(256), 0, st, f);
  else if (f.dS)
    hipLaunchKernelGGL((k_dqs16<DP, false>), dim3(nqt * f.H), dim3(256), 0, st, f);
  else if (f.rope)
    hipLaunchKernelGGL((k_q16<DP, false, true>), dim3(nqt * f.H), dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL((k_q16<DP, false, false>), dim3(nqt * f.H), dim3(256), 0, st, f);
  rc = hip_check(hipGetLastError(), f.dS ? "launching k_dqs16" : "launching k_q16");
  if (rc == ATTN_OK) rc = profile_mark(st);
  return rc;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The fp16-operand backward; rope: dQ and dK rotated back in the write-back.
static attn_status_t run_f16(const float* Q, const float* K, const float* V, const float* O,
                             const float* dO, const float* LSE, const uint32_t* seg, float* dQ,
                             float* dK, float* dV, int seq_len, int n_heads, int n_kv_heads,
                             int head_dim, float scale, void* stream, int rope, float rope_base,
                             int pos_offset) {
  attn_status_t rc = check_common(seq_len, n_heads, n_kv_heads, head_dim, scale);
  if (rc != ATTN_OK) return rc;
  const void* ptrs[] = {Q, K, V, O, dO, LSE, seg, dQ, dK, dV};
  for (const void* p : ptrs)
    if (misaligned(p)) return fail(ATTN_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
  if (seq_len == 0) return ATTN_OK;
  const int dp = padded_dim(head_dim);
  const long long Sp = ((long long)seq_len + 127) / 128 * 128;

  const long long nblk = ((long long)seq_len + 31) / 32;
  const size_t qbytes = (size_t)n_heads * Sp * dp * 2, kbytes = (size_t)n_kv_heads * Sp * dp * 2;
  size_t off = 0;
  const size_t off_D = off; off += align256((size_t)seq_len * n_heads * 4);
  const size_t off_L2 = off; off += align256((size_t)seq_len * n_heads * 4);
  const size_t off_min = off; off += align256((size_t)nblk * 4);
  const size_t off_max = off; off += align256((size_t)nblk * 4);
  const size_t off_slot = off; off += align256((size_t)(nblk + 1) * 8);
  size_t off_x[4];  // Qh, dOh, Kh, Vh
  for (int i = 0; i < 4; ++i) {
    off_x[i] = off;
    off += align256(i < 2 ? qbytes : kbytes);
  }
  // k_kv16 splits a group's heads over workgroups (partial dK, dV through a
  // workspace slice each, added by k_sumparts).  Paired tiles (plain causal)
  // carry equal work, so the splits stop at one round of resident workgroups
  // (one per CU, two up to 64 columns): more rounds only add partial sums.
  // Under a document mask the key tiles' work differs widely, and the splits
  // go on to ~1024 workgroups, which balance it (measured at S=4096 and S=16384)
  const bool pair = seg == nullptr;
  const int g = n_heads / n_kv_heads;
  const int nkt = (seq_len + 127) / 128;
  const long long kv_blocks = (long long)(pair ? (nkt + 1) / 2 : nkt) * n_kv_heads;
  long long target = 1024;
  if (pair) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 256;
    target = (long long)ncu * (dp <= 64 ? 2 : 1);
  }
  int splits = 1;
  while (kv_blocks * splits < target && g % (2 * splits) == 0) splits *= 2;
  const size_t off_part = off;
  if (splits > 1) off += align256((size_t)2 * splits * seq_len * n_kv_heads * head_dim * 4);
  // the dS/scale tiles of every (query block, key block) pair up to the
  // causal bound (a document mask uses fewer slots), 2 KiB per pair and head,
  // within the scratch limit; beyond it the query-major pass forms dS again
  const long long ds_pairs = nblk * (nblk + 1) / 2;
  bool store_ds = ds_pairs <= scratch_limit() / (n_heads * 2048ll);
  const size_t off_ds = off;
  const size_t ds_bytes = store_ds ? align256((size_t)ds_pairs * n_heads * 2048) : 0;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipMemPool_t pool;
  rc = device_pool(&pool);
  if (rc != ATTN_OK) return rc;
  void* ws = nullptr;
  hipError_t e = hipMallocFromPoolAsync(&ws, off + ds_bytes, pool, st);
  if (e == hipErrorOutOfMemory && store_ds) {
    // no room for the dS tiles: the query-major pass forms dS again instead
    (void)hipGetLastError();  // the failed allocation is not a launch error
    store_ds = false;
    e = hipMallocFromPoolAsync(&ws, off, pool, st);
  }
  rc = hip_check(e, "hipMallocFromPoolAsync(workspace)");
  if (rc != ATTN_OK) return rc;
  char* w = static_cast<char*>(ws);
  auto half_at = [&](int i) { return reinterpret_cast<_Float16*>(w + off_x[i]); };

  F16Args f;
  f.Qh = half_at(0); f.dOh = half_at(1); f.Kh = half_at(2); f.Vh = half_at(3);
  f.LSE = LSE; f.seg = seg; f.dQ = dQ; f.dK = dK; f.dV = dV;
  f.D = reinterpret_cast<float*>(w + off_D);
  f.blk_min = reinterpret_cast<const uint32_t*>(w + off_min);
  f.blk_max = reinterpret_cast<const uint32_t*>(w + off_max);
  f.LSE2 = reinterpret_cast<const float*>(w + off_L2);
  f.slot_off = reinterpret_cast<const long long*>(w + off_slot);
  f.meta_bytes = (uint32_t)(off_slot + (size_t)(nblk + 1) * 8 - off_min);
  f.meta_max = (uint32_t)(off_max - off_min);
  f.meta_slot = (uint32_t)(off_slot - off_min);
  f.dS = store_ds ? reinterpret_cast<_Float16*>(w + off_ds) : nullptr;
  f.S = seq_len; f.Sp = (int)Sp; f.H = n_heads; f.KV = n_kv_heads; f.d = head_dim; f.scale = scale;
  f.pair = pair;
  f.splits = splits;
  f.kv_work = (int)(kv_blocks * splits);
  f.part = splits > 1 ? reinterpret_cast<float*>(w + off_part) : nullptr;
  f.rope = rope;
  f.rope_pos = pos_offset;
  f.rope_base = (double)rope_base;
  CvtArgs c;
  c.Q = Q; c.dO = dO; c.K = K; c.V = V;
  c.LSE = LSE;
  c.LSE2 = reinterpret_cast<float*>(w + off_L2);
  c.Qh = half_at(0); c.dOh = half_at(1); c.Kh = half_at(2); c.Vh = half_at(3);
  c.S = seq_len; c.Sp = (int)Sp; c.H = n_heads; c.KV = n_kv_heads; c.d = head_dim;

  rc = launch_prep(seg, seq_len, reinterpret_cast<uint32_t*>(w + off_min),
                   reinterpret_cast<uint32_t*>(w + off_max), reinterpret_cast<long long*>(w + off_slot), st);
  if (rc == ATTN_OK) {
    switch (dp) {
      case 32: rc = launch_f16<32>(f, c, O, dO, st); break;
      case 64: rc = launch_f16<64>(f, c, O, dO, st); break;
      case 96: rc = launch_f16<96>(f, c, O, dO, st); break;
      case 128: rc = launch_f16<128>(f, c, O, dO, st); break;
      case 192: rc = launch_f16<192>(f, c, O, dO, st); break;
      default: rc = launch_f16<256>(f, c, O, dO, st); break;
    }
  }
  attn_status_t rc2 = hip_check(hipFreeAsync(ws, st), "hipFreeAsync(workspace)");
  return rc != ATTN_OK ? rc : rc2;
}

extern "C" attn_status_t attn_bwd_f16(const float* Q, const float* K, const float* V, const float* O,
                                      const float* dO, const float* LSE, const uint32_t* seg,
                                      float* dQ, float* dK, float* dV, int seq_len, int n_heads,
                                      int n_kv_heads, int head_dim, float scale, void* stream) {
  clear_error();
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  return run_f16(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                 scale, stream, 0, 0.f, 0);
}

extern "C" attn_status_t attn_bwd_f16_rope(const float* Q, const float* K, const float* V,
                                           const float* O, const float* dO, const float* LSE,
                                           const uint32_t* seg, float* dQ, float* dK, float* dV,
                                           int seq_len, int n_heads, int n_kv_heads, int head_dim,
                                           float scale, float rope_base, int pos_offset,
                                           void* stream) {
  clear_error();
  if (!Q || !K || !V || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (!(rope_base > 0.f) || !isfinite(rope_base))
    return fail(ATTN_ERR_INVALID_ARG, "rope_base must be positive and finite (got %g)", (double)rope_base);
  if (pos_offset < 0) return fail(ATTN_ERR_INVALID_ARG, "pos_offset must be >= 0 (got %d)", pos_offset);
  if (seq_len > 0 && (long long)pos_offset + seq_len - 1 > 0x7fffffffll)
    return fail(ATTN_ERR_INVALID_ARG, "pos_offset + seq_len exceeds 2^31");
  return run_f16(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, seq_len, n_heads, n_kv_heads, head_dim,
                 scale, stream, 1, rope_base, pos_offset);
}
