// synth_fill.hip -- device-side writer of seeded synthetic expert blobs.
//
// Input generation only (no MoE arithmetic).  Implements counter-based SplitMix64
// (Steele, Lea & Flood, OOPSLA 2014: word i of the stream keyed k is
// mix64(k + (i+1) * 0x9E3779B97F4A7C15)) and writes, for each expert, the same bytes
// as synth.expert_blob() on the host:
//   code planes : byte j = byte (j mod 8), little-endian, of word j/8 of the plane's stream;
//   sb planes   : pair p = (bf16 scale, bf16 bias) from word p: the high 24 bits give
//                 u_s, the low 24 bits u_b; value = lo + span * (u * 2^-24) evaluated as two
//                 float32 roundings (multiply, then add), then round-to-nearest-even to bf16;
//   everything else in the blob stride is zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t expert, uint64_t tensor) {
  return mix64(mix64(seed) ^ ((layer << 32) | (expert << 8) | tensor));
}

__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct FillArgs {
  uint64_t off[6];
  uint64_t size[6];
  float s_lo, s_span, b_lo, b_span;
};

// Each step rounds to fp32 on its own, as the host generator's numpy float32 steps do: no fused
// multiply-add may merge the product and the sum.
__device__ inline uint32_t sb_pair(uint64_t key, uint64_t p, const FillArgs& a) {
#pragma clang fp contract(off)
  uint64_t w = mix64(key + (p + 1) * kGamma);
  float hi = (float)(uint32_t)(w >> 40) * 5.9604644775390625e-08f;          // 2^-24, exact
  float lo = (float)(uint32_t)(w & 0xFFFFFFull) * 5.9604644775390625e-08f;
  float s = __fadd_rn(__fmul_rn(hi, a.s_span), a.s_lo);
  float b = __fadd_rn(__fmul_rn(lo, a.b_span), a.b_lo);
  return bf16_rne(s) | (bf16_rne(b) << 16);
}

__global__ void __launch_bounds__(256) fill_kernel(uint8_t* __restrict__ dst, uint64_t stride, int n_experts,
                                                   int first_expert, int layer, uint64_t seed, FillArgs a) {
  const uint64_t words_per_blob = stride / 8;
  const uint64_t total = words_per_blob * (uint64_t)n_experts;
  for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t e = w / words_per_blob;
    const uint64_t byte = (w - e * words_per_blob) * 8;
    uint64_t val = 0;
    for (int t = 0; t < 6; ++t) {
      if (byte >= a.off[t] && byte < a.off[t] + a.size[t]) {
        const uint64_t key = stream_key(seed, (uint64_t)layer, (uint64_t)(first_expert + e), (uint64_t)t);
        const uint64_t rel = byte - a.off[t];
        if ((t & 1) == 0) {
          val = mix64(key + (rel / 8 + 1) * kGamma);
        } else {
          const uint64_t p = rel / 4;
          val = (uint64_t)sb_pair(key, p, a) | ((uint64_t)sb_pair(key, p + 1, a) << 32);
        }
        break;
      }
    }
    reinterpret_cast<uint64_t*>(dst + e * stride)[byte / 8] = val;
  }
}

}  // namespace

// Returns 0 on success, 1 on bad arguments, 2 on launch failure.
extern "C" int synth_fill_blobs(void* dst, uint64_t stride, int n_experts, int first_expert, int layer,
                                uint64_t seed, const void* /*unused*/, const uint64_t* off, const uint64_t* size,
                                float s_lo, float s_span, float b_lo, float b_span, void* stream) {
  if (!dst || !off || !size || n_experts < 0 || first_expert < 0 || stride % 256 != 0) return 1;
  FillArgs a;
  for (int t = 0; t < 6; ++t) {
    a.off[t] = off[t];
    a.size[t] = size[t];
    if (off[t] % 8 != 0 || size[t] % 8 != 0 || off[t] + size[t] > stride) return 1;
  }
  a.s_lo = s_lo; a.s_span = s_span; a.b_lo = b_lo; a.b_span = b_span;
  if (n_experts == 0) return 0;
  const uint64_t total = stride / 8 * (uint64_t)n_experts;
  uint64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, stride, n_experts, first_expert, layer, seed, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
