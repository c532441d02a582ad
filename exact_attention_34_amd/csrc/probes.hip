// Achievable-peak probes of the chip (libattn_probes.so, measurement code,
// not part of the attention path).  The roofline of the tutorial "Chapter 3
// Advanced principles: performance model and numerical stability" (section
// 3.0.3) divides a kernel's rate by the machine's peak; besides the published
// peaks, the benchmark divides by what these loops reach on the same chip:
//
//   * mfma_bf16_loop: independent chains of v_mfma_f32_32x32x16_bf16 on every
//     SIMD (the prefill's matrix op), operands that vary per lane and per
//     step so that the data toggles as real data does;
//   * exp2_loop: independent chains x <- 2^-x of the transcendental unit (the
//     softmax's v_exp_f32), values in the probabilities' range;
//   * random_read: whole 4 KiB blocks read at random block ids by 2,048
//     persistent waves with two blocks in flight each, with the non-temporal
//     hint -- the access pattern of paged decode, without its arithmetic.
//
// Every kernel writes one value per thread so that nothing is optimised
// away.  The host entry points check their arguments and only enqueue.
#include "common.h"

namespace {

using attn::f32x16;
using attn::u32x4;

// A 32-bit mix of two ints (an xorshift-multiply hash): per-lane operands.
__device__ inline uint32_t mix(uint32_t x, uint32_t y) {
  x ^= y * 0x9E3779B9u;
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  return x;
}

// bf16 pairs with exponents near 1 (|x| in [0.5, 2)), random signs and
// mantissas: realistic operands for the matrix core.
__device__ inline uint32_t bf16_pair(uint32_t h) {
  const uint32_t lo = 0x3F00u | (h & 0x80FFu);
  const uint32_t hi = 0x3F00u | ((h >> 16) & 0x80FFu);
  return lo | (hi << 16);
}

constexpr int kChains = 4;   // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_bf16_loop(int iters, float* out) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[s][e] = bf16_pair(mix(tid, 8 * s + e));
      b[s][e] = bf16_pair(mix(tid, 8 * s + e + 4));
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  // two steps per iteration; the second pairs each chain with the other A
  // operand, so consecutive products of a chain see different data
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = attn::BF16::mma32(a[c & 1], b[c >> 1], acc[c]);
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = attn::BF16::mma32(a[(c & 1) ^ 1], b[c >> 1], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[tid] = s;
}

constexpr int kExpChains = 8;

__global__ __launch_bounds__(256) void exp2_loop(int iters, float* out) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = (float)(mix(tid, c) & 1023u) * (1.0f / 1024.0f);
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) s += x[c];
  out[tid] = s;
}

// Wave w reads blocks ids[w], ids[w + W], ... (W waves), each 4 KiB as four
// coalesced 1 KiB load instructions (lane l takes bytes 1024 j + 16 l .. + 15
// of instruction j).  The next block's loads are issued before the current
// one is consumed.
__global__ __launch_bounds__(64) void random_read(const char* buf, const int32_t* ids, int n_ids,
                                                  uint32_t* out) {
  const int w = blockIdx.x, W = gridDim.x, lane = threadIdx.x;
  uint32_t acc = 0;
  auto load = [&](int i, u32x4* v) {
    const char* p = buf + (int64_t)ids[i] * 4096 + lane * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load((const u32x4*)(p + 1024 * j));
  };
  u32x4 cur[4], nxt[4];
  int i = w;
  if (i < n_ids) load(i, cur);
  for (; i < n_ids; i += W) {
    if (i + W < n_ids) load(i + W, nxt);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= cur[j][0] ^ cur[j][1] ^ cur[j][2] ^ cur[j][3];
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
  }
  out[w * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// out: blocks * 256 floats of device memory.  Work: blocks * 4 waves *
// iters * 8 products * 32,768 FLOP.  Returns 0 or a hipError_t value.
int attn_probe_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_bf16_loop, dim3(blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

// out: blocks * 256 floats.  Work: blocks * 256 lanes * iters * 8 exp2.
int attn_probe_exp2(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(exp2_loop, dim3(blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

// buf: device memory of buf_bytes; ids: device [n_ids] int32, each in
// [0, buf_bytes / 4096) (the caller's guarantee); out: waves * 64 uint32.
// Reads n_ids * 4 KiB.
int attn_probe_random_read(const void* buf, size_t buf_bytes, const int32_t* ids, int n_ids,
                           uint32_t* out, int waves, void* stream) {
  if (buf == nullptr || ids == nullptr || out == nullptr || n_ids <= 0 || waves <= 0 ||
      buf_bytes < 4096 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(random_read, dim3(waves), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     (const char*)buf, ids, n_ids, out);
  return (int)hipGetLastError();
}

}  // extern "C"
