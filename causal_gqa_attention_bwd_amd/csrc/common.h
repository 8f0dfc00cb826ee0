// common.h -- device helpers shared by the fp32 kernels (attnbwd.hip) and the
// fp16-operand kernels (attnbwd_f16.hip), and the library's internal host
// helpers.  Everything here is internal to libattnbwd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---------------------------------------------------------------------------
// RoPE backward in the epilogues (page "llm.istanbul --
// 10_backward_attention.wgsl", kernels rope_q_backward / rope_k_backward):
// the pair of columns (2p, 2p+1) of a row at position pos turns back by
// angle = pos * base^(-2p/d): (g0, g1) -> (g0 c + g1 s, -g0 s + g1 c).  The
// angle and its sine and cosine are taken in fp64 (positions reach 2^31; an
// fp32 angle would be off by ~1e-3 rad at a few thousand).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rope_freq(int col, int d, double base) {
  return pow(base, -2.0 * (double)(col >> 1) / (double)d);
}
// This column's value after the backward rotation, from its own value and its
// pair partner's.
__device__ __forceinline__ float rope_back(float mine, float partner, int col, long long pos,
                                           double freq) {
  double sn, cs;
  sincos((double)pos * freq, &sn, &cs);
  return (col & 1) ? (float)(-(double)partner * sn + (double)mine * cs)
                   : (float)((double)mine * cs + (double)partner * sn);
}
// ---------------------------------------------------------------------------
// Direct buffer->LDS loads.  Each lane's 16 (or 4) bytes land at the wave's
// LDS base + 16 (or 4) * lane; the global source of every lane is free, which
// the kernels use for padding and zero fill: a lane whose offset lies beyond
// the buffer range deposits zeros without touching memory.
// ---------------------------------------------------------------------------
#define ATTN_BUF_OOB 0x80000000u        // beyond every buffer range used here
#define ATTN_BUF_WORD3 0x00020000       // raw buffer, 32-bit data format
#define ATTN_CPOL_NT 2                  // cache policy of a buffer access: non-temporal

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A raw buffer over `bytes` bytes at p for an epilogue's reads and writes:
// a load at an offset at or past the end reads zero and a store there is
// dropped (the hardware range check), so ragged rows and columns need no
// divergent branch around them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, ATTN_BUF_WORD3);
}
__device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Buffer resource of `nbytes` bytes at `base` (nbytes = 0: every load reads zeros).
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
  r.w = ATTN_BUF_WORD3;
  return r;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct buffer->LDS loads (16 or 4 bytes per lane; lane i's data lands at
// lds + i * size).  Issued from inline assembly so that the compiler does not
// treat every later LDS read as possibly overlapping these writes and wait for
// them: ordering is explicit instead -- every reader of a tile passes a
// tile_barrier (s_waitcnt vmcnt(0) + s_barrier) issued after the tile's loads,
// and no buffer is refilled before all waves have passed a barrier after
// their last read of it.  M0 carries the LDS address and is restored.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t voff, uint32_t lds_byte) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds_byte)), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t voff, uint32_t lds_byte) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds_byte)), "v"(voff), "s"(r)
      : "memory");
}
// dma16 for data read once (non-temporal: the caches need not keep it).
__device__ __forceinline__ void dma16_nt(const i32x4& r, uint32_t voff, uint32_t lds_byte) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane((int)lds_byte)), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t voff, const void* lds) {
  dma16(r, voff, lds_addr(lds));
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t voff, const void* lds) {
  dma4(r, voff, lds_addr(lds));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads it does not wait for outstanding global
// loads, so direct-to-LDS loads of the next tile stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait for all of this wave's outstanding memory operations (the current
// tile's direct-to-LDS loads among them), then a workgroup barrier: the tile is
// complete in LDS and every wave has finished with the previous tile.  The
// wait is the compiler's own s_waitcnt, so it also knows that every load it
// issued before has landed and adds no later waits for them.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
  asm volatile("s_barrier" ::: "memory");
}

// Head served by block b of a (tile, head) grid, grouping the heads of one KV
// group on one XCD: workgroups are dispatched round-robin over the 8 XCDs, so
// blocks b, b+8, b+16, ... share an L2; when H is a multiple of 8 they get
// heads x*(H/8) .. x*(H/8) + H/8 - 1 of XCD slot x = b % 8, i.e. whole groups.
__device__ __forceinline__ int xcd_head(int r, int H) {
  if (H % 8 != 0) return r;
  return (r % 8) * (H / 8) + r / 8;
}

// The mirror n - 1 - first of tile `first` among n tiles, which a paired block
// serves after `first`, or -1 (unpaired, or the middle tile of an odd n).  A
// tile and its mirror together carry the same causal work for every first.
__device__ __forceinline__ int mirror_tile(int first, int n, int pair) {
  const int mirror = n - 1 - first;
  return (pair && mirror != first) ? mirror : -1;
}

// ---------------------------------------------------------------------------
// Internal host helpers (defined in attnbwd.hip; hidden from the library's
// exported symbols).
// ---------------------------------------------------------------------------
#define ATTN_INTERNAL __attribute__((visibility("hidden")))

// Set the calling thread's error text and return st.
ATTN_INTERNAL attn_status_t fail(attn_status_t st, const char* fmt, ...);
// Clear the calling thread's error text (start of every entry point).
ATTN_INTERNAL void clear_error();
// ATTN_ERR_HIP with the HIP error text when e is not hipSuccess.
ATTN_INTERNAL attn_status_t hip_check(hipError_t e, const char* what);
// Argument checks shared by every backward entry point.
ATTN_INTERNAL attn_status_t check_common(int S, int H, int KV, int d, float scale);
ATTN_INTERNAL bool misaligned(const void* p);
// head_dim rounded up to the next supported tile width (32, 64, 96, 128, 192, 256).
ATTN_INTERNAL int padded_dim(int d);
// The library's stream-ordered memory pool of the current device.
ATTN_INTERNAL attn_status_t device_pool(hipMemPool_t* out);
// The most bytes of stored tiles one call may take (attn_set_scratch_limit).
ATTN_INTERNAL long long scratch_limit();
// Record one profile event on st when the measurement hooks are on; `first`
// opens the record of a new call.
ATTN_INTERNAL attn_status_t profile_mark(hipStream_t st, bool first = false);
// k_prep: per 32-row query block seg min / max (and the tile slot offsets).
ATTN_INTERNAL attn_status_t launch_prep(const uint32_t* seg, int S, uint32_t* blk_min,
                                        uint32_t* blk_max, long long* slot_off, hipStream_t st);
// k_rowdot: D[r] = dO[r, :] . O[r, :] for rows [0, rows) of two [rows, d] tensors.
ATTN_INTERNAL attn_status_t launch_rowdot(const float* O, const float* dO, float* D, long long rows,
                                          int d, hipStream_t st);
// k_sumparts: dK += sum of part[2 s], dV += sum of part[2 s + 1] over the
// splits s in order, on `rows` rows of `width` floats that sit `stride`
// floats apart (in dK, dV and each rows * stride slice of part).  rope: dK
// is then rotated back, dK = R^T (dK + sum), row r at position r + rope_pos
// (head_dim d, base rope_base).
ATTN_INTERNAL attn_status_t launch_sumparts(const float* part, int splits, long long rows, int width,
                                            long long stride, float* dK, float* dV, hipStream_t st,
                                            int rope = 0, int d = 0, int rope_pos = 0,
                                            double rope_base = 0.0);
