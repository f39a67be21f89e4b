// Index-key cache writer: quantize new index keys to e4m3fn with one fp32
// scale per token and scatter them into the paged cache.
//
// [ATOM-1473] "enable minimax m3 fp8 index cache ...", Pull request overview
// and the attention-layer diffs: the index-key cache is allocated in fp8 when
// the KV cache is fp8, and its writer is handed a key scale. The layout it
// writes is the one every indexer kernel here reads: per token, 128 e4m3fn
// bytes and scale = max|k| / 448, so the largest magnitude maps to 448.
//
// One wave per token: lane l holds dimensions 2l and 2l + 1, the wave takes
// the maximum magnitude with DPP, every lane encodes its two values and
// stores them as one 16-bit word (the wave writes the token's 128 bytes in
// one line), and lane 0 stores the scale.
#include "../../include/idxtopk.h"
#include "common.hpp"
#include "launch.hpp"

namespace idxtopk {

constexpr int CW_WG = 256;
constexpr int CW_DIM = 128;

// e4m3fn code of a finite fp32 value: nearest representable value, ties to
// the even mantissa, magnitudes above 448 saturating to 448, the sign kept.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  const float a = __uint_as_float(mag);
  uint32_t code;
  if (a > 448.0f) {
    code = 0x7Eu;
  } else if (a >= 0.015625f) {
    // normal (2^-6 and up): keep 3 mantissa bits with round-half-even on the
    // fp32 exponent|mantissa field (a carry moves into the exponent), then
    // rebias the exponent from 127 to 7
    const uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
  } else {
    // subnormal: m * 2^-9, m = round-half-even(a * 2^9) in 0..8 (8 is the
    // smallest normal, code 0x08)
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  }
  return code | sign;
}

template <bool BF16>
__global__ __launch_bounds__(CW_WG) void cache_write_kernel(const void* keys, int64_t stride, int tokens,
                                                            const int32_t* slots, uint8_t* kcache,
                                                            float* kscale) {
  const int t = blockIdx.x * (CW_WG / kWave) + uniform(static_cast<int>(threadIdx.x) / kWave);
  if (t >= tokens) return;
  // the key and its slot are loaded together; a skipped token only drops
  // its store
  const int32_t s = load_uniform(slots + t);
  const int l = lane_id();
  float x0, x1;
  if (BF16) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(keys) + t * stride)[l];
    x0 = __uint_as_float(v << 16);
    x1 = __uint_as_float(v & 0xFFFF0000u);
  } else {
    const float2 v = reinterpret_cast<const float2*>(static_cast<const float*>(keys) + t * stride)[l];
    x0 = v.x;
    x1 = v.y;
  }
  // largest magnitude of the token: non-negative floats order like their bits
  const uint32_t m0 = __float_as_uint(x0) & 0x7FFFFFFFu, m1 = __float_as_uint(x1) & 0x7FFFFFFFu;
  const uint32_t m = wave_max_u32(m0 > m1 ? m0 : m1);
  float scale = __fdiv_rn(__uint_as_float(m), 448.0f);
  if (!(scale > 0.0f)) scale = 1.0f;
  const uint32_t c = e4m3_code(__fdiv_rn(x0, scale)) | (e4m3_code(__fdiv_rn(x1, scale)) << 8);
  if (s < 0) return;
  reinterpret_cast<uint16_t*>(kcache + static_cast<int64_t>(s) * CW_DIM)[l] = static_cast<uint16_t>(c);
  if (l == 0) kscale[s] = scale;
}

int launch_cache_write(const void* keys, bool bf16, int64_t stride, int tokens, const int32_t* slots,
                       uint8_t* kcache, float* kscale, hipStream_t stream) {
  if (tokens == 0) return 0;
  const dim3 grid(static_cast<unsigned>((tokens + CW_WG / kWave - 1) / (CW_WG / kWave)));
  (void)hipGetLastError();
  if (bf16)
    hipLaunchKernelGGL(cache_write_kernel<true>, grid, dim3(CW_WG), 0, stream, keys, stride, tokens, slots,
                       kcache, kscale);
  else
    hipLaunchKernelGGL(cache_write_kernel<false>, grid, dim3(CW_WG), 0, stream, keys, stride, tokens, slots,
                       kcache, kscale);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---------------------------------------------------------------------------
// bf16 index cache ([ATOM-1473] Pull request overview: with a KV cache that
// is not fp8 the index cache takes the model's dtype): keys stored as bf16,
// 256 bytes per token, no scale.
// ---------------------------------------------------------------------------

// bf16 pattern of a finite fp32 value, rounded to nearest with ties to the
// even pattern: adding 0x7FFF plus the bit that becomes the last kept one
// carries into bit 16 exactly when the dropped half is above one half, or
// one half with an odd kept part.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sixteen threads per token, eight dimensions each: one 16-byte store.
// bf16 input is copied as it is.
template <bool BF16_IN>
__global__ __launch_bounds__(CW_WG) void cache_write_bf16_kernel(const void* keys, int64_t stride, int tokens,
                                                                 const int32_t* slots, uint16_t* kcache) {
  const int i = blockIdx.x * CW_WG + threadIdx.x;
  const int t = i >> 4, part = i & 15;
  if (t >= tokens) return;
  const int32_t slot = slots[t];
  if (slot < 0) return;
  uint4 out;
  if (BF16_IN) {
    out = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(keys) + t * stride + 8 * part);
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(keys) + t * stride + 8 * part);
    const float4 x = src[0], y = src[1];
    out.x = bf16_bits(x.x) | (bf16_bits(x.y) << 16);
    out.y = bf16_bits(x.z) | (bf16_bits(x.w) << 16);
    out.z = bf16_bits(y.x) | (bf16_bits(y.y) << 16);
    out.w = bf16_bits(y.z) | (bf16_bits(y.w) << 16);
  }
  *reinterpret_cast<uint4*>(kcache + static_cast<int64_t>(slot) * CW_DIM + 8 * part) = out;
}

int launch_cache_write_bf16(const void* keys, bool bf16_in, int64_t stride, int tokens, const int32_t* slots,
                            uint16_t* kcache, hipStream_t stream) {
  if (tokens == 0) return 0;
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(tokens) * 16 + CW_WG - 1) / CW_WG));
  (void)hipGetLastError();
  if (bf16_in)
    hipLaunchKernelGGL(cache_write_bf16_kernel<true>, grid, dim3(CW_WG), 0, stream, keys, stride, tokens, slots,
                       kcache);
  else
    hipLaunchKernelGGL(cache_write_bf16_kernel<false>, grid, dim3(CW_WG), 0, stream, keys, stride, tokens, slots,
                       kcache);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace idxtopk
